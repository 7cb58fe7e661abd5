// The onehot part of the head's gradient, taken exactly.
//
// "Training — design (ORPO, flash-CCE head, …)" §5.1 and "ORPO training —
// design", lever 1 spec (backward): the per-logit gradient is
// coef (softmax - onehot) (times sech^2(z / c) under a softcap c).  Its
// softmax part is spread over every vocabulary entry and goes through the
// bf16 gradient tiles and the two contractions; its onehot part is one entry
// per row, of size |coef| sech^2 at the row's target.  Rounded to bf16 with
// the rest, that entry would carry an error of up to 2^-9 of itself, which
// depends on the target's softmax value (so on h) and adds up over rows
// instead of averaging out.  So the gradient tiles hold coef * softmax only,
// and the onehot part is applied here in fp32:
//   dh_i  = -t_i W_{y_i}                     (before the chunk contractions
//                                              accumulate into dh)
//   dW_v -= sum_{i : y_i = v} t_i h_i          (after the chunks wrote dW)
// with t_i = coef_i sech^2(z_{i,y_i} / c) (coef_i without a cap).  The dW sum
// runs over each target's rows in ascending row order: the rows are grouped
// by target with a stable radix sort of (target, row) pairs, integer
// histograms and prefix sums (no floating-point atomics), so results are
// deterministic.
#include "cce_device.hpp"
#include "cce_launch.hpp"

namespace cce {

__device__ __forceinline__ float bf16_f32(u16 b) { return __builtin_bit_cast(float, (unsigned)b << 16); }

// Element d of head row v: bf16 W, or the quantised head's value
// s q + b rounded to bf16 (as the dequantised chunks hold it).
template <bool QUANT>
__device__ __forceinline__ float head_elem(const u16* __restrict__ W, const QuantW& q, int D,
                                           int v, int d) {
  if (!QUANT) return bf16_f32(W[(size_t)v * D + d]);
  const int per = 32 / q.bits, words = D / per, G = D / q.group;
  const unsigned word = q.Wq[(size_t)v * words + d / per];
  const unsigned c = (word >> (q.bits * (d % per))) & ((1u << q.bits) - 1u);
  const float s = bf16_f32(q.scale[(size_t)v * G + d / q.group]);
  const float b = bf16_f32(q.bias[(size_t)v * G + d / q.group]);
  return bf16_f32(to_bf16(fmaf(s, (float)c, b)));
}

// One wave per row: t_i, dh_i = -t_i W_{y_i} (0 for a row without a target in
// [0, V)), and the sort input (key y_i, or V for a row whose t_i is 0; value i).
// vec: D % 8 == 0 and 16-byte aligned W and dh rows (8 columns a lane).
template <bool QUANT>
__global__ __launch_bounds__(256) void k_target_dh(const u16* __restrict__ H,
                                                   const u16* __restrict__ W, QuantW q,
                                                   const int* __restrict__ y,
                                                   const float* __restrict__ coef, int M, int V,
                                                   int D, float softcap, bool vec,
                                                   float* __restrict__ dh,
                                                   float* __restrict__ tc, int* __restrict__ key,
                                                   int* __restrict__ val) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int yy = y[row];
  const bool has = yy >= 0 && yy < V;
  float t = has ? coef[row] : 0.f;
  if (has && t != 0.f && softcap > 0.f) {
    // sech^2 of the capped target logit: z = h_i . W_{y_i} (fp32 sum of exact products)
    const u16* hr = H + (size_t)row * D;
    float z = 0.f;
    for (int d = lane; d < D; d += 64) z = fmaf(bf16_f32(hr[d]), head_elem<QUANT>(W, q, D, yy, d), z);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
    const float th = tanh_scaled(z, 2.f * LOG2E / softcap);
    t *= 1.f - th * th;
  }
  float* out = dh + (size_t)row * D;
  if (!QUANT && vec) {  // 8 columns a lane: one 16-byte load of W, two 16-byte stores
    const u16* wr = W + (size_t)(t != 0.f ? yy : 0) * D;
    for (int d = 8 * lane; d < D; d += 512) {
      float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
      if (t != 0.f) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + d);
        const float nt = -t;
        o0 = make_float4(nt * bf16_f32((u16)(wv[0] & 0xffff)), nt * bf16_f32((u16)(wv[0] >> 16)),
                         nt * bf16_f32((u16)(wv[1] & 0xffff)), nt * bf16_f32((u16)(wv[1] >> 16)));
        o1 = make_float4(nt * bf16_f32((u16)(wv[2] & 0xffff)), nt * bf16_f32((u16)(wv[2] >> 16)),
                         nt * bf16_f32((u16)(wv[3] & 0xffff)), nt * bf16_f32((u16)(wv[3] >> 16)));
      }
      *reinterpret_cast<float4*>(out + d) = o0;
      *reinterpret_cast<float4*>(out + d + 4) = o1;
    }
  } else if (t != 0.f) {
    for (int d = lane; d < D; d += 64) out[d] = -t * head_elem<QUANT>(W, q, D, yy, d);
  } else {
    for (int d = lane; d < D; d += 64) out[d] = 0.f;
  }
  if (lane == 0) {
    tc[row] = t;
    key[row] = t != 0.f ? yy : V;
    val[row] = row;
  }
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort of (key, value) pairs, 8 bits a pass.  Block b holds
// entries [b R, b R + R) (R = kSortRows); per pass: each block's digit counts
// hist[d * nblk + b], an exclusive prefix over that array (digit-major, so the
// blocks of one digit follow each other in block order), and a scatter in which
// every entry goes to its digit's offset for its block plus its rank among the
// block's earlier entries with the same digit.
// ---------------------------------------------------------------------------
constexpr int kSortRows = 2048;

// Lanes of this wave whose digit equals this lane's (among the lanes with ok).
__device__ __forceinline__ unsigned long long digit_match(bool ok, int d) {
  unsigned long long m = __ballot(ok);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const unsigned long long bb = __ballot((d >> bit) & 1);
    m &= ((d >> bit) & 1) ? bb : ~bb;
  }
  return m;
}

// Digit counts of block b; each group of lanes with one digit adds its size
// once (a hot digit would otherwise take one LDS atomic per entry).
__global__ __launch_bounds__(256) void k_sort_hist(const int* __restrict__ key, int n, int shift,
                                                   int nblk, int* __restrict__ hist) {
  __shared__ int h[256];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  h[tid] = 0;
  __syncthreads();
  for (int r = 0; r < kSortRows; r += 256) {
    const int i = b * kSortRows + r + tid;
    const bool ok = i < n;
    const int d = ok ? (key[i] >> shift) & 255 : 0;
    const unsigned long long m = digit_match(ok, d);
    if (ok && (m & below) == 0ull) atomicAdd(&h[d], __popcll(m));
  }
  __syncthreads();
  hist[tid * nblk + b] = h[tid];
}

// In-place exclusive prefix sum of hist[0 .. total), one workgroup: thread t
// takes a contiguous segment, the segment sums are scanned in LDS.
__global__ __launch_bounds__(1024) void k_sort_scan(int* __restrict__ hist, int total) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (total + 1023) / 1024;
  const int s0 = tid * per, s1 = min(total, s0 + per);
  int sum = 0;
  for (int i = s0; i < s1; ++i) sum += hist[i];
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int i = s0; i < s1; ++i) {
    const int c = hist[i];
    hist[i] = run;
    run += c;
  }
}

__global__ __launch_bounds__(256) void k_sort_scatter(const int* __restrict__ key,
                                                      const int* __restrict__ val, int n,
                                                      int shift, int nblk,
                                                      const int* __restrict__ offs,
                                                      int* __restrict__ key2,
                                                      int* __restrict__ val2) {
  __shared__ int base[256];     // this block's next position per digit
  __shared__ int wcnt[4][256];  // entries per (wave, digit) in the current round
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  base[tid] = offs[tid * nblk + b];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < kSortRows; r += 256) {
#pragma unroll
    for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
    __syncthreads();
    const int i = b * kSortRows + r + tid;
    const bool ok = i < n;
    const int k = ok ? key[i] : 0;
    const int d = (k >> shift) & 255;
    const unsigned long long m = digit_match(ok, d);  // lanes of this wave with this digit
    const int rk = __popcll(m & below);
    if (ok && rk == 0) wcnt[w][d] = __popcll(m);
    __syncthreads();
    if (ok) {
      int pos = base[d] + rk;
      for (int q = 0; q < w; ++q) pos += wcnt[q][d];
      key2[pos] = k;
      val2[pos] = val[i];
    }
    __syncthreads();
    base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// The whole sort in one workgroup, in LDS (about 148 KB), for n <= kSortSmall:
// the same passes (digit counts, prefix over digits, stable scatter by ballot
// ranks), ping-ponging between two LDS copies; the result is written once.
constexpr int kSortSmall = 8192;

__global__ __launch_bounds__(1024) void k_sort_small(const int* __restrict__ key,
                                                     const int* __restrict__ val, int n, int bits,
                                                     int* __restrict__ key_out,
                                                     int* __restrict__ val_out) {
  __shared__ int kbuf[2][kSortSmall], vbuf[2][kSortSmall];
  __shared__ int hist[256];       // counts, then the running position of each digit
  __shared__ int wcnt[16 * 256];  // entries per (wave, digit) in one round
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int i = tid; i < n; i += 1024) {
    kbuf[0][i] = key[i];
    vbuf[0][i] = val[i];
  }
  int cur = 0;
  for (int shift = 0; shift < bits; shift += 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int r = 0; r < n; r += 1024) {
      const int i = r + tid;
      const bool ok = i < n;
      const int d = ok ? (kbuf[cur][i] >> shift) & 255 : 0;
      const unsigned long long m = digit_match(ok, d);
      if (ok && (m & below) == 0ull) atomicAdd(&hist[d], __popcll(m));
    }
    __syncthreads();
    {  // exclusive prefix over the 256 digits: a scan in each of 4 waves, then the waves
      int c = 0, inc = 0;
      if (tid < 256) {
        c = hist[tid];
        inc = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(inc, o);
          if (lane >= o) inc += v;
        }
        if (lane == 63) wcnt[w] = inc;
      }
      __syncthreads();
      if (tid < 256) {
        int base = 0;
        for (int q = 0; q < w; ++q) base += wcnt[q];
        hist[tid] = base + inc - c;
      }
    }
    __syncthreads();
    for (int r = 0; r < n; r += 1024) {
      for (int q = tid; q < 16 * 256; q += 1024) wcnt[q] = 0;
      __syncthreads();
      const int i = r + tid;
      const bool ok = i < n;
      const int k = ok ? kbuf[cur][i] : 0;
      const int d = (k >> shift) & 255;
      const unsigned long long m = digit_match(ok, d);
      const int rk = __popcll(m & below);
      if (ok && rk == 0) wcnt[w * 256 + d] = __popcll(m);
      __syncthreads();
      if (ok) {
        int pos = hist[d] + rk;
        for (int q = 0; q < w; ++q) pos += wcnt[q * 256 + d];
        kbuf[cur ^ 1][pos] = k;
        vbuf[cur ^ 1][pos] = vbuf[cur][i];
      }
      __syncthreads();
      if (tid < 256) {
        int add = 0;
        for (int q = 0; q < 16; ++q) add += wcnt[q * 256 + tid];
        hist[tid] += add;
      }
      __syncthreads();
    }
    cur ^= 1;
  }
  for (int i = tid; i < n; i += 1024) {
    key_out[i] = kbuf[cur][i];
    val_out[i] = vbuf[cur][i];
  }
}

// dW[v, :] -= sum_{i : y_i = v} t_i h_i, from the sorted (target, row) pairs, in
// two passes over fixed windows of kTW sorted positions (columns in strips of
// 256, one per thread):
//   window pass: the window's rows are split into pieces (maximal runs of one
//     target); each piece's sum, in row order, is formed from the window's h
//     values loaded all at once.  A piece that is a whole target's run is
//     applied to dW here; the first piece, if its target's run started in an
//     earlier window, goes to F[window] (for a window inside one run, the whole
//     window's sum); the last piece, if its run starts here and continues
//     past the window, goes to L[window].
//   carry pass: for each run that starts in window w and continues, L[w] plus
//     F of the following windows, in window order, applied to dW.
// Every run's sum has a fixed order, so results are deterministic.
constexpr int kTW = 64;

__global__ __launch_bounds__(256) void k_target_dw_win(const int* __restrict__ key,
                                                       const int* __restrict__ val, int n, int V,
                                                       const float* __restrict__ tc,
                                                       const u16* __restrict__ H, int D,
                                                       float* __restrict__ dW,
                                                       float* __restrict__ F,
                                                       float* __restrict__ Lc) {
  __shared__ int s_key[kTW + 2];  // [0]: the key before the window, [kTW + 1]: after
  __shared__ int s_row[kTW];
  __shared__ float s_t[kTW];
  __shared__ float s_sum[kTW][256];
  __shared__ int s_ps[kTW + 1];
  __shared__ int s_np, s_nv;
  const int win = blockIdx.x, tid = threadIdx.x;
  const int col = blockIdx.y * 256 + tid;
  const int p0 = win * kTW, len = min(kTW, n - p0);
  if (tid < kTW) {
    const int p = p0 + tid;
    const bool in = tid < len;
    const int k = in ? key[p] : V;
    s_key[tid + 1] = k;
    s_row[tid] = in && k < V ? val[p] : 0;
    s_t[tid] = in && k < V ? tc[val[p]] : 0.f;
  } else if (tid == kTW) {
    s_key[0] = p0 > 0 ? key[p0 - 1] : -1;
  } else if (tid == kTW + 1) {
    s_key[kTW + 1] = (len == kTW && p0 + kTW < n) ? key[p0 + kTW] : -1;
  }
  __syncthreads();
  if (tid < kTW) {  // pieces among the positions holding a target (sentinels sort last)
    const int k = s_key[tid + 1];
    const bool valid = k < V;  // positions past len hold V
    const bool head = valid && (tid == 0 || k != s_key[tid]);
    const unsigned long long hm = __ballot(head);
    const int nv = __popcll(__ballot(valid));
    if (head) s_ps[__popcll(hm & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) {
      const int np = __popcll(hm);
      s_ps[np] = nv;
      s_np = np;
      s_nv = nv;
    }
  }
  __syncthreads();
  const int np = s_np, nv = s_nv;
  if (np == 0) return;
  // this column's h values of the window's rows, all loads issued together
  float hv[kTW];
#pragma unroll
  for (int r = 0; r < kTW; ++r)
    hv[r] = (r < nv && col < D) ? bf16_f32(H[(size_t)s_row[r] * D + col]) : 0.f;
  {
    float acc = 0.f;
    int j = 0;
#pragma unroll
    for (int r = 0; r < kTW; ++r) {
      if (r < nv) {
        if (r > 0 && s_key[r + 1] != s_key[r]) {
          s_sum[j][tid] = acc;
          ++j;
          acc = 0.f;
        }
        acc = fmaf(s_t[r], hv[r], acc);
      }
    }
    s_sum[j][tid] = acc;
  }
  if (col >= D) return;
  const bool first_before = s_key[1] == s_key[0];
  const bool last_after = nv == kTW && s_key[kTW] == s_key[kTW + 1];
  // whole runs: dW rows loaded in batches of 8, then updated
  const int j0 = first_before ? 1 : 0;
  const int j1 = (last_after && !(np == 1 && first_before)) ? np - 1 : np;
  {
    float old[kTW];
#pragma unroll
    for (int e = 0; e < kTW; ++e)
      if (j0 + e < j1) old[e] = dW[(size_t)s_key[s_ps[j0 + e] + 1] * D + col];
#pragma unroll
    for (int e = 0; e < kTW; ++e)
      if (j0 + e < j1) dW[(size_t)s_key[s_ps[j0 + e] + 1] * D + col] = old[e] - s_sum[j0 + e][tid];
  }
  if (first_before) F[(size_t)win * D + col] = s_sum[0][tid];
  if (last_after && !(np == 1 && first_before)) Lc[(size_t)win * D + col] = s_sum[np - 1][tid];
}

__global__ __launch_bounds__(256) void k_target_dw_carry(const int* __restrict__ key, int n,
                                                         int V, int D,
                                                         const float* __restrict__ F,
                                                         const float* __restrict__ Lc,
                                                         float* __restrict__ dW) {
  __shared__ int s_last;
  const int win = blockIdx.x, tid = threadIdx.x, col = blockIdx.y * 256 + tid;
  const int p0 = win * kTW;
  if (p0 + kTW >= n) return;  // a run continuing past the window needs a next one
  const int k = key[p0 + kTW - 1];
  if (k >= V || key[p0 + kTW] != k) return;                         // the last run ends here
  if (key[p0] == k && p0 > 0 && key[p0 - 1] == k) return;           // it started earlier
  // the run goes through windows win + 1 .. last: window w + 1 continues it when
  // both its first and its last position hold k (keys are sorted)
  float acc = Lc[(size_t)win * D + (col < D ? col : 0)];
  for (int w0 = win + 1;; w0 += 64) {
    if (tid == 0) s_last = -1;
    __syncthreads();
    if (tid < 64) {
      const int w = w0 + tid;
      const int q = w * kTW + kTW;  // first position after window w
      const bool ends = q >= n || key[q - 1] != k || key[q] != k;
      const unsigned long long e = __ballot(ends);
      if (tid == 0 && e != 0ull) s_last = w0 + __builtin_ctzll(e);
    }
    __syncthreads();
    const int last = s_last;
    const int w1 = last >= 0 ? last : w0 + 63;
    if (col < D) {
      float f[64];
#pragma unroll
      for (int e = 0; e < 64; ++e) f[e] = (w0 + e <= w1) ? F[(size_t)(w0 + e) * D + col] : 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (w0 + e <= w1) acc += f[e];
    }
    if (last >= 0) break;
    __syncthreads();
  }
  if (col < D) dW[(size_t)k * D + col] -= acc;
}

hipError_t launch_target_dh(const BwdArgs& a, hipStream_t st) {
  const dim3 grid((a.M + 3) / 4);
  // 16-byte rows of W and dh: the bf16 head's fast path (a.vec: D % 8 == 0, W aligned)
  const bool vec = a.vec && (reinterpret_cast<uintptr_t>(a.dh) & 15u) == 0;
  if (a.q.Wq)
    CCE_TIMED(KN_TARGET_DH, 0.0, st,
              hipLaunchKernelGGL(k_target_dh<true>, grid, dim3(256), 0, st, a.H, a.W, a.q, a.y,
                                 a.coef, a.M, a.V, a.D, a.softcap, vec, a.dh, a.tc, a.skey[0],
                                 a.sval[0]));
  else
    CCE_TIMED(KN_TARGET_DH, 0.0, st,
              hipLaunchKernelGGL(k_target_dh<false>, grid, dim3(256), 0, st, a.H, a.W, a.q, a.y,
                                 a.coef, a.M, a.V, a.D, a.softcap, vec, a.dh, a.tc, a.skey[0],
                                 a.sval[0]));
  return hipGetLastError();
}

hipError_t launch_target_dw(const BwdArgs& a, hipStream_t st) {
  const int n = a.M;
  const int nblk = (n + kSortRows - 1) / kSortRows;
  int bits = 0;
  while (bits < 31 && (a.V >> bits) != 0) ++bits;  // keys are in [0, V]
  int cur = 0;
  if (n <= kSortSmall) {
    CCE_TIMED(KN_SORT, 0.0, st,
              hipLaunchKernelGGL(k_sort_small, dim3(1), dim3(1024), 0, st, a.skey[0], a.sval[0],
                                 n, bits, a.skey[1], a.sval[1]));
    cur = 1;
    bits = 0;  // done
  }
  for (int shift = 0; shift < bits; shift += 8) {
    CCE_TIMED(KN_SORT, 0.0, st,
              hipLaunchKernelGGL(k_sort_hist, dim3(nblk), dim3(256), 0, st, a.skey[cur], n, shift,
                                 nblk, a.shist));
    CCE_TIMED(KN_SORT, 0.0, st,
              hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(1024), 0, st, a.shist, 256 * nblk));
    CCE_TIMED(KN_SORT, 0.0, st,
              hipLaunchKernelGGL(k_sort_scatter, dim3(nblk), dim3(256), 0, st, a.skey[cur],
                                 a.sval[cur], n, shift, nblk, a.shist, a.skey[cur ^ 1],
                                 a.sval[cur ^ 1]));
    cur ^= 1;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((n + kTW - 1) / kTW, (a.D + 255) / 256);
  CCE_TIMED(KN_TARGET_DW, 0.0, st,
            hipLaunchKernelGGL(k_target_dw_win, grid, dim3(256), 0, st, a.skey[cur], a.sval[cur],
                               n, a.V, a.tc, a.H, a.D, a.dW, a.tF, a.tL));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CCE_TIMED(KN_TARGET_DW, 0.0, st,
            hipLaunchKernelGGL(k_target_dw_carry, grid, dim3(256), 0, st, a.skey[cur], n, a.V,
                               a.D, a.tF, a.tL, a.dW));
  return hipGetLastError();
}

}  // namespace cce
