// Exact-attention backward for gfx950, by recomputation.
//
// Method: the forward saved only O and one log-sum-exp per row; the backward
// recomputes S and P block by block instead of reading an N x N matrix
// ("FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness", reading notes (hackmd), §Algorithm › Recomputation; the
// backward's IO matches the forward's, §IO Complexity Analysis › proof sketch).
// The gradient itself is the chain rule through S = scale Q K^T, P = softmax(S),
// O = P V: with D_i = rowsum(dO o O)_i,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Kernels (same stream):
//   bwd_prep:     D and LSE * log2(e) per row; clears the f32 dQ accumulator.
//   bwd_main:     one workgroup per (instance, 128-key block); 4 waves x 32 keys.
//                 dK and dV of its keys stay in registers across the loop over
//                 32-query tiles; dQ partials are added to the f32 accumulator.
//   bwd_dq_store: dQ = scale * accumulator, rounded to bf16.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

struct BwdKParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dq_acc;
  float* delta;
  float* lse2;
  int64_t sb, sh, sn;
  int B, H, N;
  float c;      // scale * log2(e)
  float scale;
  int causal;
  const int32_t* key_len;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  int bs;
  int n_kblocks;
};

constexpr int kBwdKeys = 128;   // keys per workgroup
constexpr int kBwdQ = 32;       // queries per inner tile

// ------------------------------------------------------------------------------ prep

// One row per D/8 threads: D = sum_i dO_i O_i (f32), lse2 = LSE log2(e) (+inf when
// the row has no key so that recomputed probabilities are 0), dQ accumulator = 0.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdKParams p) {
  constexpr int TPR = D / 8;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + tid / TPR;
  const int sub = tid % TPR;
  const int64_t total = (int64_t)p.B * p.H * p.N;
  float acc = 0.f;
  if (row < total) {
    const int64_t inst = row / p.N;
    const int n = (int)(row - inst * p.N);
    const int b = (int)(inst / p.H), h = (int)(inst - (int64_t)b * p.H);
    const int64_t off = (int64_t)b * p.sb + (int64_t)h * p.sh + (int64_t)n * p.sn + 8 * sub;
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.o + off);
    const bf16x8 dv = *reinterpret_cast<const bf16x8*>(p.dout + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)ov[i], (float)dv[i], acc);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(p.dq_acc + row * D + 8 * sub) = z;
    *reinterpret_cast<f32x4*>(p.dq_acc + row * D + 8 * sub + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < total && sub == 0) {
    p.delta[row] = acc;
    const float l = p.lse[row];
    p.lse2[row] = (l == kNegInf) ? kPosInf : l * kLog2e;
  }
}

// ------------------------------------------------------------------------------ main

template <int D, bool SPARSE>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdKParams p) {
  constexpr int QP = D + 8;         // row-major Q / dO tile stride
  constexpr int TP = kBwdQ + 4;     // transposed Q / dO tile stride
  constexpr int SP = kBwdKeys + 8;  // dS tile stride ([query][key])
  constexpr int KTP = kBwdKeys + 8; // K^T stride ([dim][key])
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int QGROUPS = kBwdQ * D / 8 / 256;     // (4 queries x 2 dims) groups per thread
  constexpr int KGROUPS = kBwdKeys * D / 8 / 256;  // (4 keys x 2 dims) groups per thread
  static_assert(QGROUPS >= 1 && KGROUPS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) bf16 sQ[kBwdQ * QP];
  __shared__ __attribute__((aligned(16))) bf16 sdO[kBwdQ * QP];
  __shared__ __attribute__((aligned(16))) bf16 sQt[D * TP];
  __shared__ __attribute__((aligned(16))) bf16 sdOt[D * TP];
  __shared__ __attribute__((aligned(16))) bf16 sdS[kBwdQ * SP];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * KTP];
  __shared__ __attribute__((aligned(16))) float sL[kBwdQ];
  __shared__ __attribute__((aligned(16))) float sDl[kBwdQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_kblocks, inst, rank);
  const int kb = rank;  // causal: the lowest key blocks see the most queries; they go first
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = p.q + base;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;
  const bf16* dOh = p.dout + base;
  const int k0 = kb * kBwdKeys;
  const int kw0 = k0 + 32 * wave;  // this wave's 32 keys
  const int mykey = kw0 + l32;     // the key of this lane's MFMA column
  const int64_t rowbase = (int64_t)inst * N;

  int kv_len = N;
  if (!SPARSE && p.key_len) kv_len = min(max(p.key_len[b], 0), N);

  // The query tiles this key block visits.
  int n_qt, qt_begin = 0, cbeg = 0;
  if (SPARSE) {
    const int kbs = k0 / p.bs;
    cbeg = p.col_ptr[kbs];
    n_qt = (p.col_ptr[kbs + 1] - cbeg) * (p.bs / kBwdQ);
  } else if (k0 >= kv_len) {
    n_qt = 0;
  } else {
    qt_begin = p.causal ? k0 / kBwdQ : 0;
    n_qt = (N + kBwdQ - 1) / kBwdQ - qt_begin;
  }
  auto tile_q0 = [&](int t) -> int {
    if (SPARSE) {
      const int tpb = p.bs / kBwdQ;
      return p.row_idx[cbeg + t / tpb] * p.bs + (t - (t / tpb) * tpb) * kBwdQ;
    }
    return (qt_begin + t) * kBwdQ;
  };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }

  if (n_qt > 0) {
    // This wave's K and V as B operands of S = Q K^T and dP = dO V^T: lane
    // column = mykey; slot group g of k-step kk holds dims [16 kk + 8 g, +8).
    bf16x8 kf[NKK], vf[NKK];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int64_t off = (int64_t)mykey * p.sn + 16 * kk + 8 * g;
      kf[kk] = mykey < N ? *reinterpret_cast<const bf16x8*>(Kh + off) : __builtin_bit_cast(bf16x8, zero4);
      vf[kk] = mykey < N ? *reinterpret_cast<const bf16x8*>(Vh + off) : __builtin_bit_cast(bf16x8, zero4);
    }
    // K^T of the whole key block, for dQ = dS K.
#pragma unroll
    for (int i = 0; i < KGROUPS; ++i) {
      const int gi = tid + 256 * i, kq = gi / (D / 2), dc = gi - kq * (D / 2);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 4 * kq + j;
        w[j] = key < N ? *reinterpret_cast<const uint32_t*>(Kh + (int64_t)key * p.sn + 2 * dc) : 0u;
      }
      u32x2 xs, ys;
      split_pairs4(w[0], w[1], w[2], w[3], xs, ys);
      *reinterpret_cast<u32x2*>(&sKt[(2 * dc) * KTP + 4 * kq]) = xs;
      *reinterpret_cast<u32x2*>(&sKt[(2 * dc + 1) * KTP + 4 * kq]) = ys;
    }

    // dQ work split: D = 128: wave w owns dims [32 w, 32 w + 32) over all 128 keys;
    // D = 64: dims 32 (w & 1), keys [64 (w >> 1), +64).
    constexpr int DQ_KSTEPS = (D == 128) ? 8 : 4;
    const int dq_db = (D == 128) ? wave : (wave & 1);
    const int dq_k0 = (D == 128) ? 0 : 64 * (wave >> 1);

    for (int t = 0; t < n_qt; ++t) {
      const int q0 = tile_q0(t);
      // Stage Q_i and dO_i (row-major and transposed), lse2_i and D_i.
#pragma unroll
      for (int i = 0; i < QGROUPS; ++i) {
        const int gi = tid + 256 * i, qq = gi / (D / 2), dc = gi - qq * (D / 2);
        uint32_t wq[4], wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qi = q0 + 4 * qq + j;
          const int64_t off = (int64_t)qi * p.sn + 2 * dc;
          wq[j] = qi < N ? *reinterpret_cast<const uint32_t*>(Qh + off) : 0u;
          wd[j] = qi < N ? *reinterpret_cast<const uint32_t*>(dOh + off) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *reinterpret_cast<uint32_t*>(&sQ[(4 * qq + j) * QP + 2 * dc]) = wq[j];
          *reinterpret_cast<uint32_t*>(&sdO[(4 * qq + j) * QP + 2 * dc]) = wd[j];
        }
        u32x2 xs, ys;
        split_pairs4(wq[0], wq[1], wq[2], wq[3], xs, ys);
        *reinterpret_cast<u32x2*>(&sQt[(2 * dc) * TP + 4 * qq]) = xs;
        *reinterpret_cast<u32x2*>(&sQt[(2 * dc + 1) * TP + 4 * qq]) = ys;
        split_pairs4(wd[0], wd[1], wd[2], wd[3], xs, ys);
        *reinterpret_cast<u32x2*>(&sdOt[(2 * dc) * TP + 4 * qq]) = xs;
        *reinterpret_cast<u32x2*>(&sdOt[(2 * dc + 1) * TP + 4 * qq]) = ys;
      }
      if (tid < kBwdQ) {
        const int qi = q0 + tid;
        sL[tid] = qi < N ? p.lse2[rowbase + qi] : kPosInf;
        sDl[tid] = qi < N ? p.delta[rowbase + qi] : 0.f;
      }
      __syncthreads();

      // S = Q_i K_w^T and dP = dO_i V_w^T (rows = queries, columns = this wave's keys).
      f32x16 sacc, dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.f;
        dpacc[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sQ[l32 * QP + 16 * kk + 8 * g]);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&sdO[l32 * QP + 16 * kk + 8 * g]);
        sacc = mfma_bf16(aq, kf[kk], sacc);
        dpacc = mfma_bf16(ad, vf[kk], dpacc);
      }

      // P = 2^(c S - lse2), dS = P (dP - D). Register r is query q0 + 8 (r/4) + 4 g + r%4.
      const bool need_mask =
          !SPARSE && ((p.causal && q0 < kw0 + 31) || (kw0 + 32 > kv_len) || (q0 + kBwdQ > N));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&sL[8 * j + 4 * g]);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(&sDl[8 * j + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          float pr = fast_exp2(fmaf(sacc[r], p.c, -lv[i]));
          if (need_mask) {
            const int qi = q0 + 8 * j + 4 * g + i;
            const bool ok = mykey < kv_len && qi < N && (!p.causal || mykey <= qi);
            if (!ok) pr = 0.f;
          }
          sacc[r] = pr;
          dpacc[r] = pr * (dpacc[r] - dv[i]);
        }
      }

      // P and dS as B operands (column = key, K = queries): k-step s covers queries
      // 16 s + {4g..4g+3, 8+4g..8+4g+3}, i.e. registers 8 s .. 8 s + 7.
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        pb[s] = pack_bf16x8(sacc[8 * s + 0], sacc[8 * s + 1], sacc[8 * s + 2], sacc[8 * s + 3],
                            sacc[8 * s + 4], sacc[8 * s + 5], sacc[8 * s + 6], sacc[8 * s + 7]);
        dsb[s] = pack_bf16x8(dpacc[8 * s + 0], dpacc[8 * s + 1], dpacc[8 * s + 2], dpacc[8 * s + 3],
                             dpacc[8 * s + 4], dpacc[8 * s + 5], dpacc[8 * s + 6], dpacc[8 * s + 7]);
      }

      // dV^T += dO^T P and dK^T += Q^T dS (rows = dims, columns = this wave's keys).
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* ap = &sdOt[(db * 32 + l32) * TP + 16 * s + 4 * g];
          const bf16* aq = &sQt[(db * 32 + l32) * TP + 16 * s + 4 * g];
          const bf16x8 a_do = concat_bf16x4(*reinterpret_cast<const bf16x4*>(ap),
                                            *reinterpret_cast<const bf16x4*>(ap + 8));
          const bf16x8 a_q = concat_bf16x4(*reinterpret_cast<const bf16x4*>(aq),
                                           *reinterpret_cast<const bf16x4*>(aq + 8));
          dvacc[db] = mfma_bf16(a_do, pb[s], dvacc[db]);
          dkacc[db] = mfma_bf16(a_q, dsb[s], dkacc[db]);
        }

      // dS to LDS as [query][key] for dQ.
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sdS[(8 * (r >> 2) + 4 * g + (r & 3)) * SP + 32 * wave + l32] = (bf16)dpacc[r];
      __syncthreads();

      // dQ_i[:, dims] += dS_i K[keys, dims]: A = dS rows (query), B = K^T rows (dim),
      // slot group g of k-step ks holds keys [16 ks + 8 g, +8).
      f32x16 dqacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) dqacc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DQ_KSTEPS; ++ks) {
        const int kc = dq_k0 + 16 * ks + 8 * g;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sdS[l32 * SP + kc]);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&sKt[(dq_db * 32 + l32) * KTP + kc]);
        dqacc = mfma_bf16(a, bk, dqacc);
      }
      float* dqrow = p.dq_acc + (rowbase + q0) * D + dq_db * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qo = 8 * (r >> 2) + 4 * g + (r & 3);
        if (q0 + qo < N) unsafeAtomicAdd(dqrow + (int64_t)qo * D, dqacc[r]);
      }
      // The next tile's staging only touches buffers that every wave finished
      // reading before the barrier above; sdS is rewritten only after the next
      // tile's first barrier.
    }
  }

  // dK = scale dK^T^T, dV: lane column = mykey, register r = dim 32 db + 8 (r/4) + 4 g + r%4.
  if (mykey < N) {
    bf16* dkrow = p.dk + base + (int64_t)mykey * p.sn;
    bf16* dvrow = p.dv + base + (int64_t)mykey * p.sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dkacc[db][4 * j] * p.scale, dkacc[db][4 * j + 1] * p.scale);
        wk[1] = pack_bf16x2(dkacc[db][4 * j + 2] * p.scale, dkacc[db][4 * j + 3] * p.scale);
        wv[0] = pack_bf16x2(dvacc[db][4 * j], dvacc[db][4 * j + 1]);
        wv[1] = pack_bf16x2(dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
        *reinterpret_cast<u32x2*>(dkrow + db * 32 + 8 * j + 4 * g) = wk;
        *reinterpret_cast<u32x2*>(dvrow + db * 32 + 8 * j + 4 * g) = wv;
      }
  }
}

// ------------------------------------------------------------------------------ dQ store

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_store_kernel(BwdKParams p) {
  const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8 elements each
  const int64_t total = (int64_t)p.B * p.H * p.N * (D / 8);
  if (chunk >= total) return;
  const int64_t row = chunk / (D / 8);
  const int c8 = (int)(chunk - row * (D / 8)) * 8;
  const int64_t inst = row / p.N;
  const int n = (int)(row - inst * p.N);
  const int b = (int)(inst / p.H), h = (int)(inst - (int64_t)b * p.H);
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(p.dq_acc + row * D + c8);
  const f32x4 a1 = *reinterpret_cast<const f32x4*>(p.dq_acc + row * D + c8 + 4);
  u32x4 w;
  w[0] = pack_bf16x2(a0[0] * p.scale, a0[1] * p.scale);
  w[1] = pack_bf16x2(a0[2] * p.scale, a0[3] * p.scale);
  w[2] = pack_bf16x2(a1[0] * p.scale, a1[1] * p.scale);
  w[3] = pack_bf16x2(a1[2] * p.scale, a1[3] * p.scale);
  *reinterpret_cast<u32x4*>(p.dq + (int64_t)b * p.sb + (int64_t)h * p.sh + (int64_t)n * p.sn + c8) = w;
}

// ------------------------------------------------------------------------------ launcher

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  BwdKParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<const bf16*>(a.o);
  p.dout = static_cast<const bf16*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<bf16*>(a.dq);
  p.dk = static_cast<bf16*>(a.dk);
  p.dv = static_cast<bf16*>(a.dv);
  p.dq_acc = a.dq_acc;
  p.delta = a.delta;
  p.lse2 = a.lse2;
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.B = a.B;
  p.H = a.H;
  p.N = a.N;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.causal = a.causal;
  p.key_len = a.key_len;
  p.col_ptr = a.col_ptr;
  p.row_idx = a.row_idx;
  p.bs = a.block_size;
  p.n_kblocks = (a.N + kBwdKeys - 1) / kBwdKeys;
  const bool sparse = a.col_ptr != nullptr;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const dim3 block(256);

  const int rows_per_wg = 256 / (a.d / 8);
  const dim3 grid_prep((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  timer_begin("fa_bwd_prep", s);
  if (a.d == 128) bwd_prep_kernel<128><<<grid_prep, block, 0, s>>>(p);
  else bwd_prep_kernel<64><<<grid_prep, block, 0, s>>>(p);
  timer_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const dim3 grid_main((unsigned)(a.B * a.H * p.n_kblocks));
  timer_begin("fa_bwd_main", s);
  if (a.d == 128) {
    if (sparse) bwd_main_kernel<128, true><<<grid_main, block, 0, s>>>(p);
    else bwd_main_kernel<128, false><<<grid_main, block, 0, s>>>(p);
  } else {
    if (sparse) bwd_main_kernel<64, true><<<grid_main, block, 0, s>>>(p);
    else bwd_main_kernel<64, false><<<grid_main, block, 0, s>>>(p);
  }
  timer_end(s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t chunks = rows * (a.d / 8);
  const dim3 grid_store((unsigned)((chunks + 255) / 256));
  timer_begin("fa_bwd_dq_store", s);
  if (a.d == 128) bwd_dq_store_kernel<128><<<grid_store, block, 0, s>>>(p);
  else bwd_dq_store_kernel<64><<<grid_store, block, 0, s>>>(p);
  timer_end(s);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ block lists

// One workgroup: per-row (CSR) and per-column (CSC) lists of the nonzero blocks
// of an nb x nb mask (nb <= 1024), indices in increasing order.
__global__ __launch_bounds__(1024) void block_lists_kernel(const uint8_t* mask, int nb, int32_t* row_ptr,
                                                           int32_t* col_idx, int32_t* col_ptr,
                                                           int32_t* row_idx) {
  __shared__ int32_t rcount[1024], ccount[1024], rstart[1025], cstart[1025];
  const int tid = threadIdx.x;
  for (int i = tid; i < nb; i += 1024) {
    int rc = 0, cc = 0;
    for (int j = 0; j < nb; ++j) {
      rc += mask[(int64_t)i * nb + j] != 0;
      cc += mask[(int64_t)j * nb + i] != 0;
    }
    rcount[i] = rc;
    ccount[i] = cc;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < nb; ++i) {
      rstart[i] = acc;
      acc += rcount[i];
    }
    rstart[nb] = acc;
  } else if (tid == 64) {
    int acc = 0;
    for (int i = 0; i < nb; ++i) {
      cstart[i] = acc;
      acc += ccount[i];
    }
    cstart[nb] = acc;
  }
  __syncthreads();
  for (int i = tid; i <= nb; i += 1024) {
    row_ptr[i] = rstart[i];
    col_ptr[i] = cstart[i];
  }
  for (int i = tid; i < nb; i += 1024) {
    int rp = rstart[i], cp = cstart[i];
    for (int j = 0; j < nb; ++j) {
      if (mask[(int64_t)i * nb + j] != 0) col_idx[rp++] = j;
      if (mask[(int64_t)j * nb + i] != 0) row_idx[cp++] = j;
    }
  }
}

hipError_t launch_block_lists(const uint8_t* mask, int nb, int32_t* row_ptr, int32_t* col_idx,
                              int32_t* col_ptr, int32_t* row_idx, hipStream_t s) {
  timer_begin("fa_block_lists", s);
  block_lists_kernel<<<dim3(1), dim3(1024), 0, s>>>(mask, nb, row_ptr, col_idx, col_ptr, row_idx);
  timer_end(s);
  return hipGetLastError();
}

}  // namespace fa
