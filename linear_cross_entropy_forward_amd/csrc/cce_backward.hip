// Backward of the flash-CCE head.
//
// "Training — design (ORPO, flash-CCE head, …)" §5.1 (the analytic backward
// recomputes the logits from the saved per-row LSE and forms
// g (onehot - softmax); backward skips of near-zero softmax) and "ORPO training
// — design", lever 1 spec (backward).  With coef = -dL/dlogp:
//   G[i, v] = coef_i (softmax(i, v) - [v = y_i]),  dh = G W,  dW = G^T h.
//
// The vocabulary is walked in chunks of kVocabChunk entries.  Per chunk:
//   1. WT = W[chunk]^T             (bf16, zero padded)       HBM-bound
//   2. recompute z = h W[chunk]^T, G = coef (softmax - onehot), optional
//      filter / tile skip; G and G^T written as bf16 (RNE)   MFMA
//   3+4. dh (+)= G W[chunk] and dW[chunk] = G^T h, one launch  MFMA
// Every contraction is the same NT GEMM core with K contiguous in both
// operands; h^T is formed once per call.  dh accumulates across chunks in
// stream order, so no atomics are used and results are deterministic.  The
// workspace (G, G^T, WT, h^T) depends on M and D but not on V.
//
// Workspace matrices are stored BLOCKED (see DmaOperand): a matrix with R
// rows (a multiple of 256) and K columns (a multiple of 32) keeps element
// (r, k) at ((r / 256) * (K / 32) + k / 32) * 8192 + (r % 256) * 32 + k % 32,
// so every 256 x 32 slice the contractions stream is one contiguous 16 KB
// block, and every 256 x 256 tile the recompute writes is 128 KB in one piece.
#include "cce_device.hpp"
#include "cce_launch.hpp"

namespace cce {

__device__ __forceinline__ size_t blk_off(int r, int k, int nkb) {
  return ((size_t)(r >> 8) * nkb + (k >> 5)) * 8192 + (size_t)(r & 255) * 32 + (k & 31);
}

// Blocked dst (rows dst_rows, nkb blocks of 32 columns): dst(c, r) = src[r][c]
// for r < R, c < C, and 0 elsewhere for c < dst_rows, r < dst_k.  64 x 64
// tiles through LDS.
__global__ __launch_bounds__(256) void k_transpose(const u16* __restrict__ src, int R, int C,
                                                   int ld_src, u16* __restrict__ dst, int dst_rows,
                                                   int dst_k, int nkb, int vec) {
  __shared__ u16 t[64][66];
  const int r0 = blockIdx.x * 64;  // source rows = destination columns (K)
  const int c0 = blockIdx.y * 64;  // source columns = destination rows
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p;  // 512 chunks of 8 elements
    const int rr = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    u16 e[8];
    if (vec && r < R && c + 8 <= C) {
      u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)r * ld_src + c);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        e[2 * k] = (u16)(v[k] & 0xffffu);
        e[2 * k + 1] = (u16)(v[k] >> 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = (r < R && c + k < C) ? src[(size_t)r * ld_src + c + k] : (u16)0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) t[rr][cc + k] = e[k];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p;
    const int dr = q >> 3, dc = (q & 7) * 8;  // destination row (source column), column block
    const int orow = c0 + dr, ocol = r0 + dc;
    if (orow >= dst_rows || ocol >= dst_k) continue;
    unsigned w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (unsigned)t[dc + 2 * k][dr] | ((unsigned)t[dc + 2 * k + 1][dr] << 16);
    *reinterpret_cast<u32x4*>(dst + blk_off(orow, ocol, nkb)) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Recompute 256 (vocab) x 256 (token) logit tiles of the chunk and write their
// gradient tiles.  A = W rows of the chunk, B = h rows, so each lane owns one
// token (lse, coef, target in registers) and 16 vocab entries per MFMA tile.
// Persistent: P workgroups (a multiple of 8, at most one per CU) walk the
// tiles in steps of P, so the stores of one tile drain while the next tile's
// K loop runs.  At step t workgroup b takes logical tile
// P*t + (b % 8)*(P/8) + b/8 of the grouped raster, i.e. each XCD works on a
// contiguous run of tiles.
template <bool VEC, bool FILTER, bool KTAIL>
__global__ __launch_bounds__(NT, 1) void k_recompute(
    const u16* __restrict__ H, const u16* __restrict__ Wc, const int* __restrict__ y,
    const float* __restrict__ lse, const float* __restrict__ coef, int M, int D, int v0,
    int vlen, int nMt, int nvt, int P, float filter_eps, float block_eps,
    u16* __restrict__ G, u16* __restrict__ GT, int* __restrict__ flags, int nkbM, int nkbV) {
  __shared__ Smem sm;
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;
  const int ntiles = nMt * nvt;
  const int b = blockIdx.x;
  for (int base = 0; base < ntiles; base += P) {
    const int L = base + (b & 7) * (P >> 3) + (b >> 3);
    if (L >= ntiles) break;
    int mt, vt;
    raster_tile(L, nMt, nvt, 8, mt, vt);

    floatx16 acc[4][4];
    gemm_tile<VEC, false, KTAIL>(Wc + (size_t)vt * TILE * D, D, min(TILE, vlen - vt * TILE),
                                 H + (size_t)mt * TILE * D, D, min(TILE, M - mt * TILE), D, nullptr,
                                 0, sm, acc);

    const int vl0 = vt * TILE + wi * 128;  // chunk-local vocab row of this wave's first A row
    float nlse[4], cf[4];
    int off[4];
    bool any_tgt_lane = false;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = mt * TILE + wj * 128 + jj * 32 + (lane & 31);
      const bool ok = j < M;
      nlse[jj] = ok ? -lse[j] * LOG2E : 0.f;
      cf[jj] = ok ? coef[j] : 0.f;
      const int yy = ok ? y[j] : -1;
      off[jj] = (yy >= 0) ? yy - (v0 + vl0) - 4 * half : -1000000;
      const int o = (yy >= 0) ? yy - (v0 + vl0) : -1;
      any_tgt_lane |= (unsigned)o < 128u;
    }
    // softmax entries into acc; rows beyond the chunk's valid vocab become 0
    const bool vtail = vt * TILE + TILE > vlen;
    float pmax = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vbad = vtail && (vl0 + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= vlen);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float p = fast_exp2(fmaf(acc[ii][jj][r], LOG2E, nlse[jj]));
          if (vbad) p = 0.f;
          acc[ii][jj][r] = p;
          pmax = fmaxf(pmax, p);
        }
      }
    int* flag = flags + (size_t)mt * (nkbV / 8) + vt;
    if (block_eps > 0.f) {
      // skip the tile if every softmax entry is below block_eps and no token of
      // the tile has its target among the tile's vocab rows
      const bool keep_lane = pmax >= block_eps || any_tgt_lane;
      const bool keep_wave = __ballot(keep_lane) != 0ull;
      if (lane == 0) red[w] = keep_wave ? 1.f : 0.f;
      __syncthreads();
      const bool keep = (red[0] + red[1] + red[2] + red[3]) > 0.f;
      if (!keep) {
        if (tid == 0) *flag = 0;
        continue;
      }
    }
    if (tid == 0) *flag = 1;

    // The gradient tile leaves in two passes through LDS: G (token rows) and
    // G^T (vocab rows), each a contiguous 128 KB run of eight 16 KB blocks
    // written as 16-byte pieces.  g is formed from the softmax values kept in
    // acc in each pass.
    u16 (*st)[TILE + 8] = reinterpret_cast<u16 (*)[TILE + 8]>(&sm);
    const bool wave_has_tgt = __ballot(any_tgt_lane) != 0ull;
    auto grad4 = [&](int ii, int jj, int q) -> u32x2 {
      float g[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = acc[ii][jj][4 * q + e];
        const bool is_t = wave_has_tgt && (off[jj] == ii * 32 + 8 * q + e);
        if (FILTER && p < filter_eps && !is_t) p = 0.f;
        g[e] = cf[jj] * (is_t ? p - 1.f : p);
      }
      return u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    };
    // 16-byte chunk c of a 128 KB tile run: block c >> 10, row (c >> 2) & 255,
    // columns (c & 3) * 8 ..  Each 64 chunks of one store instruction form 1 KB
    // of contiguous memory (16 rows x 4 chunks); lane l takes row l % 16 and
    // chunk l / 16, so the 16 lanes served together read 16 different rows of
    // the same column, which the 264-element staging pitch puts in distinct
    // LDS banks.
    auto copy_out = [&](u16* dst) {
#pragma unroll 8
      for (int p = 0; p < 32; ++p) {
        const int c0 = tid + 256 * p;
        const int c = (c0 & ~63) | ((c0 & 15) << 2) | ((c0 >> 4) & 3);
        const int j = c >> 10, row = (c >> 2) & 255, col = j * 32 + (c & 3) * 8;
        *reinterpret_cast<u32x4*>(dst + (size_t)j * 8192 + row * 32 + (c & 3) * 8) =
            *reinterpret_cast<const u32x4*>(&st[row][col]);
      }
    };
    __syncthreads();  // every wave is done with the operand stages
    // pass 1: st[token][vocab] -> G rows mt*256.., K blocks vt*8 .. vt*8+7
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int tj = wj * 128 + jj * 32 + (lane & 31);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2*>(&st[tj][wi * 128 + ii * 32 + 8 * q + 4 * half]) = grad4(ii, jj, q);
    }
    __syncthreads();
    copy_out(G + ((size_t)mt * nkbV + vt * 8) * 8192);
    __syncthreads();
    // pass 2: st[vocab][token] -> G^T rows vt*256.., K blocks mt*8 .. mt*8+7
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int tj = wj * 128 + jj * 32 + (lane & 31);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int vr = wi * 128 + ii * 32 + 8 * q + 4 * half;  // tile-local vocab row
          const u32x2 pk = grad4(ii, jj, q);
          st[vr + 0][tj] = (u16)(pk[0] & 0xffffu);
          st[vr + 1][tj] = (u16)(pk[0] >> 16);
          st[vr + 2][tj] = (u16)(pk[1] & 0xffffu);
          st[vr + 3][tj] = (u16)(pk[1] >> 16);
        }
    }
    __syncthreads();
    copy_out(GT + ((size_t)vt * nkbM + mt * 8) * 8192);
    __syncthreads();  // staging reads done before the next tile's loads overwrite LDS
  }
}

// One fp32-output contraction C[ta*256 + i][tb*256 + j] (+)= sum_k A[i][k] B[j][k]
// over an nA x nB tile grid launched as nl workgroups; A and B are blocked
// workspace matrices (tile ta of A starts a_tile elements after A).
struct GemmProb {
  const u16* A;
  size_t a_tile;
  const u16* B;
  size_t b_tile;
  int K;
  float* C;
  int ldc, c_rows, c_cols;
  int nA, nB, nl;
  const int* kflags;  // per 256-wide K block of A tile ta: kflags[ta*fa + kb*fk]
  int fa, fk;
  int accum;  // 1: C += result, 0: C = result
};

// The dh and dW contractions of one vocab chunk in a single launch: workgroups
// [0, p0.nl) take p0 (dh, the longer K), the rest take p1 (dW).  Dispatching
// the long tiles first lets the short ones fill the tail, so the two problems
// together keep every CU busy (dh alone has too few output tiles).
template <bool SKIP>
__global__ __launch_bounds__(NT, 1) void k_grads(GemmProb p0, GemmProb p1) {
  __shared__ Smem sm;
  int b = blockIdx.x;
  const bool second = b >= p0.nl;
  const GemmProb p = second ? p1 : p0;
  if (second) b -= p0.nl;
  int ta, tb;
  if (!map_tile(b, p.nl, p.nA, p.nB, 8, ta, tb)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w & 1, wj = w >> 1, half = lane >> 5;
  floatx16 acc[4][4];
  gemm_tile<true, SKIP, false, true>(p.A + ta * p.a_tile, 0, TILE, p.B + tb * p.b_tile, 0, TILE, p.K,
                                     SKIP ? p.kflags + (size_t)ta * p.fa : nullptr, p.fk, sm, acc);
  const bool accum = p.accum != 0;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = ta * TILE + wi * 128 + ii * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (row >= p.c_rows) continue;
      float* crow = p.C + (size_t)row * p.ldc;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = tb * TILE + wj * 128 + jj * 32 + (lane & 31);
        if (col < p.c_cols) {
          if (accum) crow[col] += acc[ii][jj][r];
          else crow[col] = acc[ii][jj][r];
        }
      }
    }
}

static inline int pad8(int n) { return (n + 7) / 8 * 8; }

hipError_t launch_backward(const BwdArgs& a, hipStream_t st) {
  hipError_t e;
  const int nDt = a.Dpad / kTile;
  const int nkbM = a.Mpad / 32, nkbV = a.Vc / 32;
  // h^T, blocked [Dpad rows, Mpad columns], zero padded
  hipLaunchKernelGGL(k_transpose, dim3(a.Mpad / 64, a.Dpad / 64), dim3(256), 0, st, a.H, a.M, a.D,
                     a.D, a.HT, a.Dpad, a.Mpad, nkbM, (int)a.vec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool filt = a.filter_eps > 0.f;
  for (int v0 = 0; v0 < a.V; v0 += a.Vc) {
    const int vlen = a.V - v0 < a.Vc ? a.V - v0 : a.Vc;
    const int nvt = (vlen + kTile - 1) / kTile;
    const u16* Wc = a.W + (size_t)v0 * a.D;
    // 1. WT = W[chunk]^T, blocked [Dpad rows, Vc columns] (the first nvt*256 used)
    hipLaunchKernelGGL(k_transpose, dim3(nvt * kTile / 64, a.Dpad / 64), dim3(256), 0, st, Wc, vlen,
                       a.D, a.D, a.WT, a.Dpad, nvt * kTile, nkbV, (int)a.vec);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 2. recompute + gradient tile
    {
      const int n = a.nMt * nvt;
      const int P = pad8(n) < a.ncu8 ? pad8(n) : a.ncu8;  // persistent workgroups
#define CCE_RECOMPUTE(VEC, FILT, KT)                                                               \
  hipLaunchKernelGGL((k_recompute<VEC, FILT, KT>), dim3(P), dim3(NT), 0, st, a.H, Wc, a.y, a.lse,  \
                     a.coef, a.M, a.D, v0, vlen, a.nMt, nvt, P, a.filter_eps, a.block_eps, a.G,    \
                     a.GT, a.flags, nkbM, nkbV)
      const bool kt = a.D % BK != 0;
      if (!a.vec) {
        if (filt) CCE_RECOMPUTE(false, true, false); else CCE_RECOMPUTE(false, false, false);
      } else if (kt) {
        if (filt) CCE_RECOMPUTE(true, true, true); else CCE_RECOMPUTE(true, false, true);
      } else {
        if (filt) CCE_RECOMPUTE(true, true, false); else CCE_RECOMPUTE(true, false, false);
      }
#undef CCE_RECOMPUTE
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 3+4. dh (+)= G W[chunk] and dW[chunk] = G^T h in one launch
    //   dh: A = G (row tiles = token tiles, K = nvt*256), B = WT (row tiles = D tiles)
    //   dW: A = G^T (row tiles = chunk vocab tiles, K = Mpad), B = h^T
    {
      const bool skip = a.block_eps > 0.f;
      const int fstride = a.Vc / kTile;
      GemmProb dh{a.G, (size_t)nkbV * 8192, a.WT, (size_t)nkbV * 8192, nvt * kTile, a.dh, a.D, a.M,
                  a.D, a.nMt, nDt, pad8(a.nMt * nDt), a.flags, fstride, 1, v0 == 0 ? 0 : 1};
      GemmProb dw{a.GT, (size_t)nkbM * 8192, a.HT, (size_t)nkbM * 8192, a.Mpad,
                  a.dW + (size_t)v0 * a.D, a.D, vlen, a.D, nvt, nDt, pad8(nvt * nDt), a.flags, 1,
                  fstride, 0};
      if (skip)
        hipLaunchKernelGGL(k_grads<true>, dim3(dh.nl + dw.nl), dim3(NT), 0, st, dh, dw);
      else
        hipLaunchKernelGGL(k_grads<false>, dim3(dh.nl + dw.nl), dim3(NT), 0, st, dh, dw);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace cce
