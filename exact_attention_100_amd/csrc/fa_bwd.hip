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
// Kernels (same stream, in this order):
//   bwd_dq:    one workgroup per (instance, 128-query block), 4 waves x 32 queries;
//              it first forms D and LSE log2(e) for its rows (kept in registers and
//              written to the workspace), then keeps dQ in registers while it
//              streams the key tiles its rows see.
//   bwd_dkdv:  one workgroup per (instance, 128-key block), 4 waves x 32 keys; dK
//              and dV of its keys stay in registers while it streams the query
//              tiles that may see them, reading D and LSE log2(e) per tile.
// dQ is computed in its own pass (recomputing S and dP there) rather than
// accumulated across key blocks with atomics: each output is written once, by
// one workgroup, so the result is deterministic and no f32 accumulator is needed.
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
  float* delta;
  float* lse2;
  int64_t sb, sh, sn;
  int B, H, N;
  float c;      // scale * log2(e)
  float scale;
  int causal;
  const int32_t* key_len;
  const uint8_t* bmask;    // block-sparse: uint8 [nb][nb], row = query block
  int nb;
  int bs;
  int n_blocks;            // 128-row blocks of N
  Dropout drop;            // p8 == 0: none
};

constexpr int kBwdBlock = 128;  // keys (dK/dV pass) or queries (dQ pass) per workgroup

#ifndef FA_BWD_WAVES_PER_EU
#define FA_BWD_WAVES_PER_EU 2
#endif

// ------------------------------------------------------------------------------ dK, dV

// Query rows per tile of the dK/dV pass, per head dim.
// FA_BWD_DKDV_PIPE: the dK/dV tile as one stream of MFMAs with the softmax work in
// slices between them (1), or as separate product and softmax phases (0).
// FA_BWD_DKDV_AHEAD_D*: MFMAs whose LDS operands are in flight ahead of their use
// (one at d = 128, where more does not fit in 256 registers).
#ifndef FA_BWD_DKDV_PIPE
#define FA_BWD_DKDV_PIPE 1
#endif
#ifndef FA_BWD_DKDV_AHEAD_D128
#define FA_BWD_DKDV_AHEAD_D128 1
#endif
#ifndef FA_BWD_DKDV_AHEAD_D64
#define FA_BWD_DKDV_AHEAD_D64 2
#endif
#ifndef FA_BWD_TILE_Q_D128
#define FA_BWD_TILE_Q_D128 32
#endif
#ifndef FA_BWD_TILE_Q_D64
#define FA_BWD_TILE_Q_D64 64
#endif

// Per query tile of BRQ rows (double-buffered in LDS by direct copies, one
// barrier per tile), each wave, for its 32 keys:
//   S = Q K_w^T, dP = dO V_w^T   (A = Q / dO rows from LDS, B = K_w / V_w in VGPRs);
//   P = 2^(c S - lse2), dS = P (dP - D);
//   dV^T += dO^T P, dK^T += Q^T dS   (A = dO^T / Q^T through transposing LDS reads).
// Loads past the end are clamped to the last row: such queries have lse2 = +inf
// (P = 0) and such keys are masked (P = 0); their outputs are not stored.
// VLDS: the key block's V stays in LDS (read as the B operand of dP) instead of
// VGPRs, which keeps the d = 128 kernel within 256 registers (two waves per SIMD).
// SMASK: a block-sparse launch that also applies the causal / key-length
// element masks (without it, sparse tiles are never masked).
// DROP: dropout on P (dense and block-sparse launches), the keep bits regenerated
// from the same counters as the forward: dV takes P o Z / (1 - p) and dP is masked and scaled
// the same way before dS = P (dP - D).
template <int D, int BRQ, bool SPARSE, bool VLDS, bool SMASK = false, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FA_BWD_WAVES_PER_EU)))
void bwd_dkdv_kernel(BwdKParams p) {
  constexpr int NQB = BRQ / 32;
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int TILE = BRQ * D;
  static_assert(BRQ <= 64, "row statistics use one 64-lane copy");
  constexpr bool PIPE = FA_BWD_DKDV_PIPE && (!VLDS || NQB == 1);  // (one V row read per dP product)

  // Double buffers. The pipelined tile reads them only through inline assembly, so
  // they share one array [Q0 | dO0 | Q1 | dO1]: each lane's read addresses are then
  // computed once and a read names its buffer by the instruction's immediate offset.
  // The phased tile reads them with compiler loads and keeps separate arrays, each
  // access naming one statically (the loop is unrolled by two), so that reads of the
  // current tile do not wait for the copies of the next tile still in flight.
  __shared__ __attribute__((aligned(16))) bf16 sT[PIPE ? 4 * TILE : 8];
  __shared__ __attribute__((aligned(16))) bf16 sQ0[PIPE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) bf16 sQ1[PIPE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) bf16 sdO0[PIPE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) bf16 sdO1[PIPE ? 8 : TILE];
  bf16* const bQ0 = PIPE ? sT : sQ0;
  bf16* const bdO0 = PIPE ? sT + TILE : sdO0;
  bf16* const bQ1 = PIPE ? sT + 2 * TILE : sQ1;
  bf16* const bdO1 = PIPE ? sT + 3 * TILE : sdO1;
  __shared__ __attribute__((aligned(16))) float sL0[64];
  __shared__ __attribute__((aligned(16))) float sL1[64];
  __shared__ __attribute__((aligned(16))) float sDl0[64];
  __shared__ __attribute__((aligned(16))) float sDl1[64];
  __shared__ __attribute__((aligned(16))) bf16 sV[VLDS ? kBwdBlock * D : 8];
  // Block-sparse: the query blocks that see this key block.
  __shared__ int16_t sBlk[SPARSE ? kMaxBlocks : 1];
  __shared__ int sBlkN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_blocks, inst, rank);
  const int kb = rank;  // causal: the lowest key blocks see the most queries; they go first
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = p.q + base;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;
  const bf16* dOh = p.dout + base;
  const int k0 = kb * kBwdBlock;
  const int kw0 = k0 + 32 * wave;  // this wave's 32 keys
  const int mykey = kw0 + l32;     // the key of this lane's MFMA column
  const int64_t rowbase = (int64_t)inst * N;

  int kv_len = N;
  if (p.key_len) kv_len = min(max(p.key_len[b], 0), N);
  // The tile-independent parts of the element mask's bounds (see mask_scores), formed
  // once per lane so that no per-lane predicate stays live across the tile loop.
  const int lo_lane = mykey < kv_len ? (p.causal ? mykey : 0) - 4 * g : 0x7FFFFFFF;  // (minus q0 >= 0: no overflow)
  const int hi_lane = N - 1 - 4 * g;

  // The query tiles this key block visits (none when all its keys are past
  // kv_len: dK = dV = 0).
  int n_blk = 0;
  if constexpr (SPARSE) n_blk = kept_block_list<false>(p.bmask, p.nb, k0 / p.bs, p.causal, sBlk, &sBlkN);
  int n_qt, qt_begin = 0;
  if (k0 >= kv_len) {
    n_qt = 0;
  } else if (SPARSE) {
    n_qt = n_blk * (p.bs / BRQ);
  } else {
    qt_begin = p.causal ? k0 / BRQ : 0;
    n_qt = (N + BRQ - 1) / BRQ - qt_begin;
  }
  auto tile_q0 = [&](int t) -> int {
    if (SPARSE) {
      const int tpb = p.bs / BRQ;
      return sBlk[t / tpb] * p.bs + (t - (t / tpb) * tpb) * BRQ;
    }
    return (qt_begin + t) * BRQ;
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
    bf16x8 kf[NKK], vf[VLDS ? 1 : NKK];
    const int64_t koff = (int64_t)min(mykey, N - 1) * p.sn + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(Kh + koff + 16 * kk);
    const int wu = uniform_wave_id();
    if constexpr (VLDS) {
      // keys past the end are clamped (their P is 0)
      TileCopy<kBwdBlock, D, 4> cpv;
      cpv.init(wu, lane, p.sn);
      cpv.issue(sV, Vh, p.sn, k0, N);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) vf[kk] = *reinterpret_cast<const bf16x8*>(Vh + koff + 16 * kk);
    }

    TileCopy<BRQ, D, 4> cp;
    cp.init(wu, lane, p.sn);
    TileOffsets<D> to;
    to.init(lane);
    TileAddr<D> ta;  // (the pipelined tile's addresses in sT)
    ta.init(to, lds_address(sT));
    auto issue_tile = [&](int q0, bf16* qw, bf16* dow, float* lw, float* dlw) __attribute__((always_inline)) {
      cp.issue(qw, Qh, p.sn, q0, N);
      cp.issue(dow, dOh, p.sn, q0, N);
      if (wave == 0) vec_dma64(lw, p.lse2 + rowbase, q0, N, lane);
      if (wave == 1) vec_dma64(dlw, p.delta + rowbase, q0, N, lane);
    };

    issue_tile(tile_q0(0), bQ0, bdO0, sL0, sDl0);
    wait_vmem();
    __syncthreads();

    // Iteration t reads tile t from (qr, dor, lr, dlr) and copies tile t + 1
    // into (qw, dow, lw, dlw).
    auto iteration = [&](int t, const bf16* qr, const bf16* dor, const float* lr, const float* dlr, bf16* qw,
                         bf16* dow, float* lw, float* dlw) __attribute__((always_inline)) {
      const int q0 = tile_q0(t);
      if constexpr (!PIPE) to.refresh();
      // Prefetch the next tile into the idle buffers (the last iteration re-reads
      // its own tile); every wave finished reading them before the previous barrier.
      issue_tile(tile_q0(min(t + 1, n_qt - 1)), qw, dow, lw, dlw);

      // Dropout keep bits of this tile, bit 16 sb + r for register r of query block sb
      // (registers 4 j .. 4 j + 3 are query quad q0 + 4 g + 8 (4 sb + j)), computed
      // before the products while few registers are live.
      uint32_t keepbits = 0;
      if (DROP && !PIPE) {
        keepbits = dropout_col_bits<4 * NQB>(p.drop, mykey, q0 + 4 * g, (uint32_t)inst);
        asm volatile("" : "+v"(keepbits));
        __builtin_amdgcn_sched_barrier(0);
      }

      // Rows past N carry lse2 = +inf (P = 0) only when they exist in the loaded
      // statistics, so they are masked too. Masked entries of S become -inf, so that
      // 2^(c S - lse2) = 0 there (c > 0).
      const bool need_mask =
          (!SPARSE || SMASK) && ((p.causal && q0 < kw0 + 31) || (kw0 + 32 > kv_len) || (q0 + BRQ > N));
      // Register r of query block sb is query q0 + 4 g + off with off a compile-time
      // constant: the entry is kept iff lo <= off <= hi (the lane's key is below kv_len
      // and, when causal, at or before the query; the query is below N).
      auto mask_scores = [&](f32x16 (&s)[NQB]) __attribute__((always_inline)) {
        const RangeMask rm(lo_lane - q0, hi_lane - q0);
#pragma unroll
        for (int sb = 0; sb < NQB; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * sb + 8 * (r >> 2) + (r & 3);
            if (!rm.keep(off)) s[sb][r] = kNegInf;
          }
      };

      // A wave whose keys all follow this tile's queries (causal) or lie past kv_len
      // has P = 0 on the whole tile: its products would add nothing, so it skips them
      // (it still issues its share of the copies and meets the barrier).
      const int kw0u = k0 + 32 * wu;
      const bool idle = (!SPARSE || SMASK) && ((p.causal && q0 + BRQ - 1 < kw0u) || kw0u >= kv_len);
      if constexpr (PIPE) {
        if (!idle) {
        // One stream of MFMAs: S (NSM of them), dP (NSM), dV (NVM), dK (NVM). Each
        // MFMA's LDS operand is an inline-assembly read issued AH MFMAs ahead and
        // waited for exactly (lds_wait; with copies in flight the compiler would
        // drain every LDS read before each product). The element work runs in slices
        // between the MFMAs that do not depend on it: P = 2^(c S - lse2) between
        // the dP products, dS = P (dP - D) between the dV products, so that each
        // wave keeps its matrix core busy through its own softmax work.
        constexpr int NE = 16 * NQB;       // scores per lane
        constexpr int NG = NE / 4;         // groups of four (one 16-byte read of lse2 or D)
        constexpr int NSM = NKK * NQB;     // S products (as many dP products)
        constexpr int NVM = 2 * NQB * NDB; // dV products (as many dK products)
        constexpr int NM = 2 * NSM + 2 * NVM;
        constexpr int AH = D == 128 ? FA_BWD_DKDV_AHEAD_D128 : FA_BWD_DKDV_AHEAD_D64;
        static_assert(!VLDS || NQB == 1, "one V row read per dP product");
        // Byte offsets of this tile's buffers in sT (constants once the loop is unrolled).
        const int qoff = (int)(lds_address(qr) - lds_address(sT)), dooff = (int)(lds_address(dor) - lds_address(sT));
        uint32_t vdelta = VLDS ? lds_address(sV) - lds_address(sT) + (uint32_t)wu * (64 * D) : 0u;
        // (opaque per tile, so that the V row addresses are not hoisted into registers)
        asm volatile("" : "+s"(vdelta));
        const uint32_t lbase = lds_address(lr) + 16 * g, dbase = lds_address(dlr) + 16 * g;
        // Group G (registers 4 (G % 4) .. + 3 of query block G / 4) is exponentiated
        // after dP product sP(G) and turned into dS after dV product sD(G); its lse2 and
        // D are read two MFMAs earlier. Slice 0 of each phase is left out: the first
        // product's inputs are still in flight.
        auto sP = [](int G) { return 1 + (G * (NSM - 1)) / NG; };
        auto sD = [](int G) { return 1 + (G * (NVM - 1)) / NG; };
        int nrd = 0;  // reads issued so far in this tile (all indices fold to constants)
        bf16x8 ra[AH + 1], rb[AH + 1];
        int ia[AH + 1];
        f32x4 lq[NG], dq[NG];
        int il[NG], id[NG];
        auto fetch = [&](int m) __attribute__((always_inline)) {
          const int s = m % (AH + 1);
          if (m < NSM) {
            ra[s] = ta.read_row(qoff, m % NQB, m / NQB);
            nrd += 1;
          } else if (m < 2 * NSM) {
            const int j = m - NSM;
            ra[s] = ta.read_row(dooff, j % NQB, j / NQB);
            nrd += 1;
            if constexpr (VLDS) {
              rb[s] = lds_read_b128_asm(ta.row[j] + vdelta, 0);  // the wave's V rows
              nrd += 1;
            }
          } else if (m < 2 * NSM + NVM) {
            const int i = m - 2 * NSM;
            ra[s] = ta.read_tr(dooff, i / NDB, i % NDB);
            nrd += 2;
          } else {
            const int i = m - 2 * NSM - NVM;
            ra[s] = ta.read_tr(qoff, i / NDB, i % NDB);
            nrd += 2;
          }
          ia[s] = nrd - 1;
        };
        auto fetch_stats = [&](int m) __attribute__((always_inline)) {
#pragma unroll
          for (int G = 0; G < NG; ++G) {
            const int off = 128 * (G / 4) + 32 * (G % 4);  // floats 32 sb + 8 j, in bytes
            if (m == NSM + sP(G) - 2) {
              lq[G] = lds_read_f32x4_asm(lbase, off);
              il[G] = nrd++;
            }
            if (m == 2 * NSM + sD(G) - 2) {
              dq[G] = lds_read_f32x4_asm(dbase, off);
              id[G] = nrd++;
            }
          }
        };
        f32x16 sacc[NQB], dpacc[NQB];
#pragma unroll
        for (int sb = 0; sb < NQB; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sacc[sb][r] = 0.f;
            dpacc[sb][r] = 0.f;
          }
        bf16x8 pb[2 * NQB], dsb[2 * NQB];
        Philox rng{};
#pragma unroll
        for (int m = 0; m < AH; ++m) fetch(m);
        static_for<NM>([&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value;
          if (m + AH < NM) fetch(m + AH);
          fetch_stats(m);
          int need = ia[m % (AH + 1)];
#pragma unroll
          for (int G = 0; G < NG; ++G) {
            if (m == NSM + sP(G)) need = il[G] > need ? il[G] : need;
            if (m == 2 * NSM + sD(G)) need = id[G] > need ? id[G] : need;
          }
          lds_wait(nrd - 1 - need);
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 a = ra[m % (AH + 1)];
          if (m < NSM) {
            sacc[m % NQB] = mfma_bf16(a, kf[m / NQB], sacc[m % NQB]);
            if constexpr (DROP) {
              // Dropout keep bits of the tile (bit 16 sb + r for register r of query block
              // sb): the generator calls' rounds run between the S products, which carry
              // no other element work.
              constexpr int NCALL = NQB;  // one call per four query quads
              constexpr int NR = 10 * NCALL;
#pragma unroll
              for (int r = (m * NR) / NSM; r < ((m + 1) * NR) / NSM; ++r) {
                const int call = r / 10;
                if (r % 10 == 0) rng = dropout_col_state(p.drop, mykey, q0 + 4 * g, (uint32_t)inst, 4 * call);
                rng.round(r % 10);
                if (r % 10 == 9) keepbits |= dropout_col_bits_of(p.drop, mykey, rng, 4 * call);
              }
            }
          } else if (m < 2 * NSM) {
            const int j = m - NSM;
            if constexpr (VLDS)
              dpacc[j % NQB] = mfma_bf16(a, rb[m % (AH + 1)], dpacc[j % NQB]);
            else
              dpacc[j % NQB] = mfma_bf16(a, vf[j / NQB], dpacc[j % NQB]);
            if (j == 0 && need_mask) mask_scores(sacc);
#pragma unroll
            for (int G = 0; G < NG; ++G)
              if (j == sP(G)) {
                const int sb = G / 4, r0 = 4 * (G % 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  sacc[sb][r0 + i] = fast_exp2(fmaf(sacc[sb][r0 + i], p.c, -lq[G][i]));
                  asm volatile("" : "+v"(sacc[sb][r0 + i]));  // keeps the slice here
                }
                if (G & 1) {
                  const int h = 8 * ((G % 4) / 2);
                  const f32x16& P = sacc[sb];
                  if constexpr (DROP) {
                    // dV takes P o Z / (1 - p)
                    float pz[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) pz[k] = ((keepbits >> (16 * sb + h + k)) & 1u) ? P[h + k] * p.drop.scale : 0.f;
                    pb[G / 2] = pack_bf16x8(pz[0], pz[1], pz[2], pz[3], pz[4], pz[5], pz[6], pz[7]);
                  } else {
                    pb[G / 2] = pack_bf16x8(P[h], P[h + 1], P[h + 2], P[h + 3], P[h + 4], P[h + 5], P[h + 6], P[h + 7]);
                  }
                }
              }
          } else if (m < 2 * NSM + NVM) {
            const int i = m - 2 * NSM;
            dvacc[i % NDB] = mfma_bf16(a, pb[i / NDB], dvacc[i % NDB]);
#pragma unroll
            for (int G = 0; G < NG; ++G)
              if (i == sD(G)) {
                const int sb = G / 4, r0 = 4 * (G % 4);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  if constexpr (DROP) {
                    // dS = P (dP o Z / (1 - p) - D)
                    const float z = ((keepbits >> (16 * sb + r0 + k)) & 1u) ? p.drop.scale : 0.f;
                    dpacc[sb][r0 + k] = sacc[sb][r0 + k] * fmaf(dpacc[sb][r0 + k], z, -dq[G][k]);
                  } else {
                    dpacc[sb][r0 + k] = sacc[sb][r0 + k] * (dpacc[sb][r0 + k] - dq[G][k]);
                  }
                }
                if (G & 1) {
                  const int h = 8 * ((G % 4) / 2);
                  const f32x16& S = dpacc[sb];
                  dsb[G / 2] = pack_bf16x8(S[h], S[h + 1], S[h + 2], S[h + 3], S[h + 4], S[h + 5], S[h + 6], S[h + 7]);
                  asm volatile("" : "+v"(dsb[G / 2]));
                }
              }
          } else {
            const int i = m - 2 * NSM - NVM;
            dkacc[i % NDB] = mfma_bf16(a, dsb[i / NDB], dkacc[i % NDB]);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        }
      } else {
      // S = Q_i K_w^T and dP = dO_i V_w^T (rows = queries, columns = this wave's keys).
      f32x16 sacc[NQB], dpacc[NQB];
#pragma unroll
      for (int sb = 0; sb < NQB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[sb][r] = 0.f;
          dpacc[sb][r] = 0.f;
        }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int sb = 0; sb < NQB; ++sb) {
          bf16x8 vb;
          if constexpr (VLDS)
            vb = to.read_row(sV, wu, kk);
          else
            vb = vf[kk];
          sacc[sb] = mfma_bf16(to.read_row(qr, sb, kk), kf[kk], sacc[sb]);
          dpacc[sb] = mfma_bf16(to.read_row(dor, sb, kk), vb, dpacc[sb]);
        }

      // P = 2^(c S - lse2), dS = P (dP - D). Register r of sub-block sb is query
      // q0 + 32 sb + 8 (r/4) + 4 g + r%4.
      if (need_mask) mask_scores(sacc);
#pragma unroll
      for (int sb = 0; sb < NQB; ++sb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 lv = *reinterpret_cast<const f32x4*>(&lr[32 * sb + 8 * j + 4 * g]);
          const f32x4 dv = *reinterpret_cast<const f32x4*>(&dlr[32 * sb + 8 * j + 4 * g]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            if (DROP) {
              // In place (a second set of temporaries would not fit in the registers):
              // dS = P (dP o Z / (1 - p) - D), then the dropped P o Z / (1 - p) for dV.
              const float z = ((keepbits >> (16 * sb + r)) & 1u) ? p.drop.scale : 0.f;
              dpacc[sb][r] = fmaf(dpacc[sb][r], z, -dv[i]);
              sacc[sb][r] = fast_exp2(fmaf(sacc[sb][r], p.c, -lv[i]));
              dpacc[sb][r] *= sacc[sb][r];
              sacc[sb][r] *= z;
            } else {
              const float pr = fast_exp2(fmaf(sacc[sb][r], p.c, -lv[i]));
              sacc[sb][r] = pr;
              dpacc[sb][r] = pr * (dpacc[sb][r] - dv[i]);
            }
          }
        }

      // P and dS as B operands (column = key, K index = query): query step qs =
      // 2 sb + s covers queries 32 sb + 16 s + {4g..4g+3, 8+4g..8+4g+3}, i.e.
      // registers 8 s .. 8 s + 7 of sub-block sb.
      bf16x8 pb[2 * NQB], dsb[2 * NQB];
#pragma unroll
      for (int sb = 0; sb < NQB; ++sb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x16& P = sacc[sb];
          const f32x16& S = dpacc[sb];
          pb[2 * sb + s] = pack_bf16x8(P[8 * s], P[8 * s + 1], P[8 * s + 2], P[8 * s + 3], P[8 * s + 4],
                                       P[8 * s + 5], P[8 * s + 6], P[8 * s + 7]);
          dsb[2 * sb + s] = pack_bf16x8(S[8 * s], S[8 * s + 1], S[8 * s + 2], S[8 * s + 3], S[8 * s + 4],
                                        S[8 * s + 5], S[8 * s + 6], S[8 * s + 7]);
        }

      // dV^T += dO^T P and dK^T += Q^T dS (rows = dims, columns = this wave's keys).
#pragma unroll
      for (int qs = 0; qs < 2 * NQB; ++qs)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dvacc[db] = mfma_bf16(to.read_tr(dor, qs, db), pb[qs], dvacc[db]);
          dkacc[db] = mfma_bf16(to.read_tr(qr, qs, db), dsb[qs], dkacc[db]);
        }
      }

      wait_vmem();
      __syncthreads();
    };
    for (int t = 0; t < n_qt; t += 2) {
      iteration(t, bQ0, bdO0, sL0, sDl0, bQ1, bdO1, sL1, sDl1);
      if (t + 1 < n_qt) iteration(t + 1, bQ1, bdO1, sL1, sDl1, bQ0, bdO0, sL0, sDl0);
    }
  }

  // dK = scale (dK^T)^T, dV: lane column = mykey, register r = dim 32 db + 8 (r/4) + 4 g + r%4;
  // with the pipelined tile's single array both leave through LDS, one after the other,
  // so that each store writes whole rows.
  if constexpr (PIPE) {
    static_assert(4 * 32 * D <= 4 * TILE, "four 32-row slices fit in the tile buffers");
    __syncthreads();
    bf16* const slice = sT + uniform_wave_id() * (32 * D);
    {
      u32x2 w[NDB][4];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w[db][j][0] = pack_bf16x2(dkacc[db][4 * j] * p.scale, dkacc[db][4 * j + 1] * p.scale);
          w[db][j][1] = pack_bf16x2(dkacc[db][4 * j + 2] * p.scale, dkacc[db][4 * j + 3] * p.scale);
        }
      store_rows_via_lds<D>(slice, w, p.dk + base, p.sn, kw0, N, lane);
    }
    __builtin_amdgcn_wave_barrier();
    {
      u32x2 w[NDB][4];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w[db][j][0] = pack_bf16x2(dvacc[db][4 * j], dvacc[db][4 * j + 1]);
          w[db][j][1] = pack_bf16x2(dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
        }
      store_rows_via_lds<D>(slice, w, p.dv + base, p.sn, kw0, N, lane);
    }
  } else if (mykey < N) {
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

// ------------------------------------------------------------------------------ dQ

// Keys per tile of the dQ pass, per head dim (64 at d = 128 just fits 256 registers and
// measured 6% faster than 32 at N = 8192).
#ifndef FA_BWD_TILE_K_D128
#define FA_BWD_TILE_K_D128 64
#endif
#ifndef FA_BWD_TILE_K_DROP_D128
#define FA_BWD_TILE_K_DROP_D128 64
#endif
// FA_BWD_DQ_PIPE: the dQ tile as one stream of MFMAs with the P and dS work in slices
// between them (1), or as separate product and element phases (0).
#ifndef FA_BWD_DQ_PIPE
#define FA_BWD_DQ_PIPE 1
#endif
#ifndef FA_BWD_DQ_AHEAD_D128
#define FA_BWD_DQ_AHEAD_D128 1
#endif
#ifndef FA_BWD_DQ_AHEAD_D64
#define FA_BWD_DQ_AHEAD_D64 2
#endif
#ifndef FA_BWD_TILE_K_D64
#define FA_BWD_TILE_K_D64 64
#endif
// Dense d = 128 without dropout: the dK/dV pass as two wave groups (bwd_dkdv_pp_kernel).
#ifndef FA_BWD_DKDV_PINGPONG
#define FA_BWD_DKDV_PINGPONG 1
#endif
// Dense d = 128 without dropout: the dQ pass as two wave groups (bwd_dq_pp_kernel).
#ifndef FA_BWD_DQ_PINGPONG
#define FA_BWD_DQ_PINGPONG 1
#endif

// Per key tile of BC keys (double-buffered in LDS by direct copies), each wave,
// for its 32 queries (one query per lane column, as in the forward):
//   S^T = K Q^T, dP^T = V dO^T     (A = K / V rows from LDS, B = Q / dO in VGPRs);
//   P^T = 2^(c S^T - lse2_q), dS^T = P^T (dP^T - D_q)   (one lse2, D per lane);
//   dQ^T += K^T dS^T               (A = K^T through the transposing LDS read,
//                                   B = dS^T straight from the accumulator layout).
// Loads past the end are clamped to the last row: such keys are masked (P = 0)
// and such queries are not stored.
template <int D, int BC, bool SPARSE, bool SMASK = false, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FA_BWD_WAVES_PER_EU)))
void bwd_dq_kernel(BwdKParams p) {
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int TILE = BC * D;
  constexpr bool PIPE = FA_BWD_DQ_PIPE && NKB == 2;

  // Double buffers: one array [K0 | V0 | K1 | V1] for the pipelined tile (inline-assembly
  // reads, the buffer named by the immediate offset); separate arrays named statically
  // for the phased tile (the key-tile loop is unrolled by two), so that its compiler
  // reads of the current tile do not wait for the copies of the next.
  __shared__ __attribute__((aligned(16))) bf16 sT[PIPE ? 4 * TILE : 8];
  __shared__ __attribute__((aligned(16))) bf16 sK0[PIPE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) bf16 sK1[PIPE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV0[PIPE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV1[PIPE ? 8 : TILE];
  bf16* const bK0 = PIPE ? sT : sK0;
  bf16* const bV0 = PIPE ? sT + TILE : sV0;
  bf16* const bK1 = PIPE ? sT + 2 * TILE : sK1;
  bf16* const bV1 = PIPE ? sT + 3 * TILE : sV1;
  // Block-sparse: this query block's kept key blocks.
  __shared__ int16_t sBlk[SPARSE ? kMaxBlocks : 1];
  __shared__ int sBlkN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_blocks, inst, rank);
  const int qb = (!SPARSE && p.causal) ? (p.n_blocks - 1 - rank) : rank;  // heaviest causal rows first
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = p.q + base;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;
  const bf16* dOh = p.dout + base;
  const int q0 = qb * kBwdBlock;
  const int qrow = q0 + 32 * wave + l32;
  const int qc = min(qrow, N - 1);
  const int64_t rowbase = (int64_t)inst * N;

  // The key tiles this query block visits (as in the forward).
  int kv_len = N, n_tiles;
  if (p.key_len) kv_len = min(max(p.key_len[b], 0), N);
  if constexpr (SPARSE) {
    n_tiles = kept_block_list<true>(p.bmask, p.nb, q0 / p.bs, p.causal, sBlk, &sBlkN) * (p.bs / BC);
  } else {
    int kv_end = kv_len;
    if (p.causal) kv_end = min(kv_end, q0 + kBwdBlock);
    n_tiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  }
  auto tile_kv0 = [&](int t) -> int {
    if (SPARSE) {
      if (t >= n_tiles) return 0;
      const int tpb = p.bs / BC;
      return sBlk[t / tpb] * p.bs + (t - (t / tpb) * tpb) * BC;
    }
    return t * BC;
  };

  // This lane's query row of Q and dO as B operands (dims [16 kk + 8 g, +8)),
  // and its row statistics.
  bf16x8 qf[NKK], df[NKK];
  const int64_t qoff = (int64_t)qc * p.sn + 8 * g;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + qoff + 16 * kk);
    df[kk] = *reinterpret_cast<const bf16x8*>(dOh + qoff + 16 * kk);
  }
  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  TileCopy<BC, D, 4> cp;
  cp.init(uniform_wave_id(), lane, p.sn);
  TileOffsets<D> to;
  to.init(lane);
  TileAddr<D> ta;  // (the pipelined tile's addresses in sT)
  ta.init(to, lds_address(sT));
  auto issue_tile = [&](int kv0, bf16* kw, bf16* vw) __attribute__((always_inline)) {
    cp.issue(kw, Kh, p.sn, kv0, N);
    cp.issue(vw, Vh, p.sn, kv0, N);
  };
  issue_tile(tile_kv0(0), bK0, bV0);

  // The row statistics the recomputation needs, formed while the first tile's copies
  // are in flight: D = sum_i dO_i O_i (this lane's half of the dims, then its partner
  // lane's) and lse2 = LSE log2(e), or +inf when the row has no key so that
  // recomputed probabilities are 0. The dK/dV pass, launched after this one, reads
  // them from the workspace.
  float d_half = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.o + base + qoff + 16 * kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) d_half = fmaf((float)ov[i], (float)df[kk][i], d_half);
  }
  const float d_q = pair_sum(d_half);
  const float lse_q = p.lse[rowbase + qc];
  const float lse2_q = (lse_q == kNegInf) ? kPosInf : lse_q * kLog2e;
  if (qrow < N && g == 0) {
    p.delta[rowbase + qrow] = d_q;
    p.lse2[rowbase + qrow] = lse2_q;
  }

  wait_vmem();
  __syncthreads();

  // Iteration t reads tile t from (kr, vr) and copies tile t + 1 into (kw, vw).
  auto iteration = [&](int t, const bf16* kr, const bf16* vr, bf16* kw, bf16* vw) __attribute__((always_inline)) {
    const int kv0 = tile_kv0(t);
    if constexpr (!PIPE) to.refresh();
    issue_tile(tile_kv0(min(t + 1, n_tiles - 1)), kw, vw);

    // dS^T = P^T (dP^T - D); register r of block kb is key kv0 + 32 kb + 8 (r/4) + 4 g + r%4.
    const bool need_mask = (!SPARSE || SMASK) && ((kv0 + BC > kv_len) || (p.causal && kv0 + BC - 1 > q0 + 32 * wave));
    // Masked entries of S become -inf, so that 2^(c S - lse2) = 0 there (c > 0).
    // (A key is kept iff key <= min(kv_len - 1, qrow when causal); register r holds key
    // kv0 + 32 kb + 4 g + off with off a compile-time constant: one compare per entry.)
    auto mask_block = [&](f32x16& s, int kb) __attribute__((always_inline)) {
      const int lim = min(kv_len - 1, p.causal ? qrow : 0x3FFFFFFF) - kv0 - 32 * kb - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off > lim) s[r] = kNegInf;
      }
    };

    f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[kb][r] = 0.f;
        dpacc[kb][r] = 0.f;
      }

    // A wave whose queries all precede this tile's keys (causal), or a tile past
    // kv_len, has P = 0 everywhere: the wave skips its products (not the copies or
    // the barrier).
    const int wq = uniform_wave_id();
    const bool idle = (!SPARSE || SMASK) && ((p.causal && kv0 > q0 + 32 * wq + 31) || kv0 >= kv_len);
    if constexpr (PIPE) {
      if (!idle) {
      // One stream of MFMAs per tile, key block by key block: S^T of blocks 0 and 1
      // (NKK each), dP^T of blocks 0 and 1, then dQ (NQM). LDS operands are
      // inline-assembly reads issued AH MFMAs ahead and waited for exactly. The
      // element work of a block starts one MFMA after the products it needs:
      // P of block 0 between the S products of block 1, P of block 1 between the dP
      // products of block 0, dS of block 0 between those of block 1, and dS of
      // block 1 between the first half of the dQ products (which use block 0 only).
      constexpr int NS = NKK * NKB;            // S products (as many dP products)
      constexpr int NQM = (BC / 16) * NDB;     // dQ products
      constexpr int NM = 2 * NS + NQM;
      constexpr int AH = D == 128 ? FA_BWD_DQ_AHEAD_D128 : FA_BWD_DQ_AHEAD_D64;
      // Byte offsets of this tile's buffers in sT (constants once the loop is unrolled).
      const int koff = (int)(lds_address(kr) - lds_address(sT)), voff = (int)(lds_address(vr) - lds_address(sT));
      int nrd = 0;  // reads issued so far in this tile (folds to constants)
      bf16x8 ra[AH + 1];
      int ia[AH + 1];
      auto fetch = [&](int m) __attribute__((always_inline)) {
        const int s = m % (AH + 1);
        if (m < NS) {
          ra[s] = ta.read_row(koff, m / NKK, m % NKK);
          nrd += 1;
        } else if (m < 2 * NS) {
          ra[s] = ta.read_row(voff, (m - NS) / NKK, (m - NS) % NKK);
          nrd += 1;
        } else {
          const int i = m - 2 * NS;
          ra[s] = ta.read_tr(koff, i / NDB, i % NDB);
          nrd += 2;
        }
        ia[s] = nrd - 1;
      };
      // Element windows [w0, w0 + len) of MFMA indices and the share of slot m in it.
      auto share = [](int m, int w0, int len, int& e0, int& e1) {
        const int k = m - w0;
        e0 = (k >= 0 && k < len) ? (k * 16) / len : 0;
        e1 = (k >= 0 && k < len) ? ((k + 1) * 16) / len : 0;
      };
      bf16x8 dsb[2 * NKB];
      uint32_t dw[4 * NKB];  // dropout keep words (see the S slices)
      Philox rng{};
#pragma unroll
      for (int m = 0; m < AH; ++m) fetch(m);
      static_for<NM>([&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        if (m + AH < NM) fetch(m + AH);
        lds_wait(nrd - 1 - ia[m % (AH + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 a = ra[m % (AH + 1)];
        if (m < NS) {
          sacc[m / NKK] = mfma_bf16(a, qf[m % NKK], sacc[m / NKK]);
          if constexpr (DROP) {
            // Keep words of key block m / NKK (key quads 4 kb .. 4 kb + 3 of this lane's
            // query): that call's ten rounds run between the block's S products.
            const int kb = m / NKK, k = m % NKK;
#pragma unroll
            for (int r = (k * 10) / NKK; r < ((k + 1) * 10) / NKK; ++r) {
              if (r == 0) rng = dropout_row_state(p.drop, qrow, kv0 + 4 * g, (uint32_t)inst, 4 * kb);
              rng.round(r);
              if (r == 9) dropout_row_words_of<4 * NKB>(qrow, rng, 4 * kb, dw);
            }
          }
        }
        else if (m < 2 * NS)
          dpacc[(m - NS) / NKK] = mfma_bf16(a, df[(m - NS) % NKK], dpacc[(m - NS) / NKK]);
        else
          dqacc[(m - 2 * NS) % NDB] = mfma_bf16(a, dsb[(m - 2 * NS) / NDB], dqacc[(m - 2 * NS) % NDB]);
        // P of block kb over window (first S product of the next block or first dP
        // product) + 1 .. its end; the mask first when this tile needs it.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int w0 = (kb == 0 ? NKK : NS) + 1, len = NKK - 1;
          if (m == w0 && need_mask) mask_block(sacc[kb], kb);
          int e0, e1;
          share(m, w0, len, e0, e1);
#pragma unroll
          for (int e = e0; e < e1; ++e) {
            sacc[kb][e] = fast_exp2(fmaf(sacc[kb][e], p.c, -lse2_q));
            asm volatile("" : "+v"(sacc[kb][e]));  // keeps the slice here (no sinking to its use)
          }
        }
        // dS of block kb: block 0 between the dP products of block 1, block 1
        // between the dQ products of the first half.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int w0 = (kb == 0 ? NS + NKK : 2 * NS) + 1, len = kb == 0 ? NKK - 1 : NQM / 2 - 1;
          int e0, e1;
          share(m, w0, len, e0, e1);
#pragma unroll
          for (int e = e0; e < e1; ++e) {
            if constexpr (DROP) {
              // dS = P (dP o Z / (1 - p) - D); register e of block kb is byte e % 4 of word e / 4
              const uint32_t w = dw[4 * kb + e / 4];
              const float z = ((w >> (8 * (e % 4))) & 0xFFu) >= p.drop.p8 ? p.drop.scale : 0.f;
              dpacc[kb][e] = sacc[kb][e] * fmaf(dpacc[kb][e], z, -d_q);
            } else {
              dpacc[kb][e] = sacc[kb][e] * (dpacc[kb][e] - d_q);
            }
            if ((e & 7) == 7) {
              const int h = e - 7;
              const f32x16& S = dpacc[kb];
              dsb[2 * kb + h / 8] = pack_bf16x8(S[h], S[h + 1], S[h + 2], S[h + 3], S[h + 4], S[h + 5], S[h + 6], S[h + 7]);
              asm volatile("" : "+v"(dsb[2 * kb + h / 8]));
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      }
    } else {
    // S^T and dP^T (keys x queries).
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = mfma_bf16(to.read_row(kr, kb, kk), qf[kk], sacc[kb]);
        dpacc[kb] = mfma_bf16(to.read_row(vr, kb, kk), df[kk], dpacc[kb]);
      }

    if (need_mask)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) mask_block(sacc[kb], kb);
    // Dropout: registers 4 q4 .. 4 q4 + 3 of block kb are key quad c = 4 kb + q4
    // (keys kv0 + 4 g + 8 c .. + 3) of this lane's query.
    uint32_t dw[4 * NKB];
    if (DROP) dropout_row_words<4 * NKB>(p.drop, qrow, kv0 + 4 * g, (uint32_t)inst, dw);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t w = DROP ? dw[4 * kb + q4] : 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * q4 + c;
          const float pr = fast_exp2(fmaf(sacc[kb][r], p.c, -lse2_q));
          if (DROP) {
            const float z = ((w >> (8 * c)) & 0xFFu) >= p.drop.p8 ? p.drop.scale : 0.f;
            dpacc[kb][r] = pr * (dpacc[kb][r] * z - d_q);
          } else {
            dpacc[kb][r] = pr * (dpacc[kb][r] - d_q);
          }
        }
      }
    bf16x8 dsb[2 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x16& S = dpacc[kb];
        dsb[2 * kb + s] = pack_bf16x8(S[8 * s], S[8 * s + 1], S[8 * s + 2], S[8 * s + 3], S[8 * s + 4],
                                      S[8 * s + 5], S[8 * s + 6], S[8 * s + 7]);
      }
    }

    // dQ^T (dims x queries) += K^T dS^T: the K^T slots of k-step ks are keys
    // 16 ks + {4g..4g+3, 8+4g..8+4g+3}, those of dsb[ks].
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqacc[db] = mfma_bf16(to.read_tr(kr, ks, db), dsb[ks], dqacc[db]);
    }

    wait_vmem();
    __syncthreads();
  };
  for (int t = 0; t < n_tiles; t += 2) {
    iteration(t, bK0, bV0, bK1, bV1);
    if (t + 1 < n_tiles) iteration(t + 1, bK1, bV1, bK0, bV0);
  }

  // dQ = scale dQ^T^T: lane = query, register r = dim 32 db + 8 (r/4) + 4 g + r%4; with the
  // pipelined tile's single array it leaves through LDS so that each store writes whole rows.
  u32x2 w[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[db][j][0] = pack_bf16x2(dqacc[db][4 * j] * p.scale, dqacc[db][4 * j + 1] * p.scale);
      w[db][j][1] = pack_bf16x2(dqacc[db][4 * j + 2] * p.scale, dqacc[db][4 * j + 3] * p.scale);
    }
  if constexpr (PIPE) {
    static_assert(4 * 32 * D <= 4 * TILE, "four 32-row slices fit in the tile buffers");
    __syncthreads();
    store_rows_via_lds<D>(sT + uniform_wave_id() * (32 * D), w, p.dq + base, p.sn, q0 + 32 * wave, N, lane);
  } else if (qrow < N) {
    bf16* dqrow = p.dq + base + (int64_t)qrow * p.sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(dqrow + db * 32 + 8 * j + 4 * g) = w[db][j];
  }
}

// ------------------------------------------------------------ dK, dV, two wave groups

// The dK/dV pass with the products and the element work in different waves at any one
// time (the scheme of the two-group forward): 8 waves own 256 keys, waves w and w + 4
// share a SIMD and form two groups that run half a query tile apart, separated by
// workgroup barriers. Wave (group gr, index wg) owns the 32 keys k0 + 64 wg + 32 gr ..
//   product phase t:  dV^T += dO_{t-1}^T P(t - 1), dK^T += Q_{t-1}^T dS(t - 1),
//                     S(t) = Q_t K^T, dP(t) = dO_t V^T;
//   element phase t:  mask, P = 2^(c S - lse2), dS = P (dP - D), bf16 packing.
// The products and the element work per tile are those of bwd_dkdv_kernel, in the same
// order per accumulator, so the two kernels give the same bits. The key block's V
// (256 rows) stays in LDS; Q/dO tiles and their row statistics are triple-buffered
// (tile t - 1's are read by the products of phase t) and copied by group 0 during its
// product phase t (tile t + 1), waited for at the end of its element phase t.
constexpr int kBwdKeysPP = 256;
#ifndef FA_BWD_DKDV_PP_AHEAD
#define FA_BWD_DKDV_PP_AHEAD 2
#endif

template <int D, int BRQ>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv_pp_kernel(BwdKParams p) {
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int TILE = BRQ * D;
  static_assert(BRQ == 32, "one 32-query block per tile");
  constexpr int NSM = NKK;       // S products (as many dP products)
  constexpr int NVM = 2 * NDB;   // dV products (as many dK products)
  // [Q0 | dO0 | Q1 | dO1 | Q2 | dO2], then the key block's V.
  __shared__ __attribute__((aligned(16))) bf16 sT[6 * TILE];
  __shared__ __attribute__((aligned(16))) bf16 sV[kBwdKeysPP * D];
  __shared__ __attribute__((aligned(16))) float sL[3][64];
  __shared__ __attribute__((aligned(16))) float sDl[3][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_wave_id();
  const int gr = wave >> 2, wg = wave & 3;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_blocks, inst, rank);
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = p.q + base;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;
  const bf16* dOh = p.dout + base;
  const int k0 = rank * kBwdKeysPP;  // causal: the lowest key blocks see the most queries; they go first
  const int kw0 = k0 + 64 * wg + 32 * gr;  // this wave's 32 keys
  const int mykey = kw0 + l32;
  const int64_t rowbase = (int64_t)inst * N;
  int kv_len = N;
  if (p.key_len) kv_len = min(max(p.key_len[b], 0), N);
  const int qt_begin = p.causal ? k0 / BRQ : 0;
  const int n_qt = k0 >= kv_len ? 0 : (N + BRQ - 1) / BRQ - qt_begin;
  auto tile_q0 = [&](int t) { return (qt_begin + min(t, n_qt - 1)) * BRQ; };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }

  if (n_qt > 0) {
    // This wave's K as the B operand of S = Q K^T (lane column = mykey; slot group g of
    // k-step kk holds dims [16 kk + 8 g, +8)); its V rows are read from LDS.
    bf16x8 kf[NKK];
    const int64_t koff = (int64_t)min(mykey, N - 1) * p.sn + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(Kh + koff + 16 * kk);
    {
      TileCopy<kBwdKeysPP, D, 8> cpv;  // keys past the end are clamped (their P is 0)
      cpv.init(wave, lane, p.sn);
      cpv.issue(sV, Vh, p.sn, k0, N);
    }
    TileCopy<BRQ, D, 4> cp;
    cp.init(wg, lane, p.sn);
    TileAddr<D> ta;
    {
      TileOffsets<D> to;
      to.init(lane);
      ta.init(to, lds_address(sT));
    }
    auto qbuf = [](int j) { return 4 * TILE * j; };            // byte offsets in sT
    auto dobuf = [](int j) { return 4 * TILE * j + 2 * TILE; };
    // (opaque, so that the V row addresses are not hoisted into registers per k-step)
    uint32_t vdelta = lds_address(sV) - lds_address(sT) + (uint32_t)(2 * wg + gr) * (64 * D);
    asm volatile("" : "+s"(vdelta));
    auto issue_tile = [&](int t, int j) __attribute__((always_inline)) {
      const int q0 = tile_q0(t);
      cp.issue(sT + qbuf(j) / 2, Qh, p.sn, q0, N);
      cp.issue(sT + dobuf(j) / 2, dOh, p.sn, q0, N);
      if (wg == 0) vec_dma64(sL[j], p.lse2 + rowbase, q0, N, lane);
      if (wg == 1) vec_dma64(sDl[j], p.delta + rowbase, q0, N, lane);
    };

    f32x16 sacc, dpacc;
    bf16x8 pb[2], dsb[2];
    // Operand ring of the product phases (slot m % (AH + 1) holds product m's operands).
    // A phase's first AH reads are issued at the end of the element phase before it (PRE):
    // they read the previous tile's dO, resident since that tile's own products, and
    // arrive while the waves wait at the barrier instead of after it.
    constexpr int AH = FA_BWD_DKDV_PP_AHEAD;
    bf16x8 ra[AH + 1], rb[AH + 1];
    // Issues the LDS reads of product m of a phase over buffers j (this tile) and jp (the
    // previous one); returns how many reads that is.
    auto fetch_op = [&](int m, int j, int jp, auto dkv_flag, bool issue) __attribute__((always_inline)) {
      constexpr bool DKV = decltype(dkv_flag)::value;
      constexpr int NP = DKV ? 2 * NVM : 0;
      const int sl = m % (AH + 1);
      if (m < NP) {
        const int i = m % NVM;
        if (issue) ra[sl] = ta.read_tr(m < NVM ? dobuf(jp) : qbuf(jp), i / NDB, i % NDB);
        return 2;
      } else if (m < NP + NSM) {
        if (issue) ra[sl] = ta.read_row(qbuf(j), 0, m - NP);
        return 1;
      } else {
        const int jj = m - NP - NSM;
        if (issue) {
          ra[sl] = ta.read_row(dobuf(j), 0, jj);
          rb[sl] = lds_read_b128_asm(ta.row[jj] + vdelta, 0);
        }
        return 2;
      }
    };
    // Product phase: (DKV) dV, dK of the previous tile from buffer jp, then S, dP of this
    // tile from buffer j. Every LDS operand is an inline-assembly read issued AH products
    // ahead and waited for exactly.
    auto products = [&](int j, int jp, auto dkv_flag, auto pre_flag) __attribute__((always_inline)) {
      constexpr bool DKV = decltype(dkv_flag)::value, PRE = decltype(pre_flag)::value;
      constexpr int NP = DKV ? 2 * NVM : 0;
      constexpr int NM = NP + 2 * NSM;
      int ia[AH + 1];
      int nrd = 0;
      auto fetch = [&](int m, bool issue) __attribute__((always_inline)) {
        nrd += fetch_op(m, j, jp, dkv_flag, issue);
        ia[m % (AH + 1)] = nrd - 1;
      };
#pragma unroll
      for (int m = 0; m < AH; ++m) fetch(m, !PRE);
      static_for<NM>([&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        if (m + AH < NM) fetch(m + AH, true);
        lds_wait(nrd - 1 - ia[m % (AH + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 a = ra[m % (AH + 1)];
        if constexpr (DKV && m < NVM) {
          dvacc[m % NDB] = mfma_bf16(a, pb[m / NDB], dvacc[m % NDB]);
        } else if constexpr (m < NP) {
          constexpr int i = m - NVM;
          dkacc[i % NDB] = mfma_bf16(a, dsb[i / NDB], dkacc[i % NDB]);
        } else if constexpr (m < NP + NSM) {
          constexpr int jj = m - NP;
          sacc = mfma_bf16(a, kf[jj], jj == 0 ? f32x16{} : sacc);
        } else {
          constexpr int jj = m - NP - NSM;
          dpacc = mfma_bf16(a, rb[m % (AH + 1)], jj == 0 ? f32x16{} : dpacc);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // Element phase of tile t (register r is query q0 + 8 (r/4) + 4 g + r%4; kept iff
    // lo <= its offset <= hi, as in bwd_dkdv_kernel), stats from buffer j.
    auto elements = [&](int t, int j) __attribute__((always_inline)) {
      const int q0 = tile_q0(t);
      if ((p.causal && q0 < kw0 + 31) || (kw0 + 32 > kv_len) || (q0 + BRQ > N)) {
        const RangeMask rm(mykey < kv_len ? (p.causal ? mykey : 0) - q0 - 4 * g : 0x3FFFFFFF, N - 1 - q0 - 4 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          if (!rm.keep(off)) sacc[r] = kNegInf;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&sL[j][8 * jj + 4 * g]);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(&sDl[j][8 * jj + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * jj + i;
          sacc[r] = fast_exp2(fmaf(sacc[r], p.c, -lv[i]));
          dpacc[r] = sacc[r] * (dpacc[r] - dv[i]);
        }
      }
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int o = 8 * h8;
        pb[h8] = pack_bf16x8(sacc[o], sacc[o + 1], sacc[o + 2], sacc[o + 3], sacc[o + 4], sacc[o + 5], sacc[o + 6],
                             sacc[o + 7]);
        dsb[h8] = pack_bf16x8(dpacc[o], dpacc[o + 1], dpacc[o + 2], dpacc[o + 3], dpacc[o + 4], dpacc[o + 5],
                              dpacc[o + 6], dpacc[o + 7]);
      }
      // (keeps the phase's work inside it)
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(dsb[0]), "+v"(dsb[1]));
    };

    // Both groups run product phase t, barrier, element phase t, barrier; group 1 starts
    // one barrier later, group 0 ends with one extra barrier.
    if (gr == 0) issue_tile(0, 0);
    wait_vmem();  // (V, and tile 0 for group 0)
    __syncthreads();
    if (gr == 1) __syncthreads();
    auto tile = [&](int t, int j, auto dkv_flag) __attribute__((always_inline)) {
      // tile t in buffer j, tile t - 1 in (j + 2) % 3; tile t + 1 goes to (j + 1) % 3
      if (gr == 0) issue_tile(t + 1, (j + 1) % 3);
      products(j, (j + 2) % 3, dkv_flag, dkv_flag);  // (tiles after the first were prefetched)
      __syncthreads();
      elements(t, j);
      if (t + 1 < n_qt) {
#pragma unroll
        for (int m = 0; m < AH; ++m) fetch_op(m, (j + 1) % 3, j, Flag<true>{}, true);
      }
      if (gr == 0) wait_vmem();
      __syncthreads();
    };
    tile(0, 0, Flag<false>{});
    for (int t = 1; t < n_qt; t += 3) {
      tile(t, 1, Flag<true>{});
      if (t + 1 < n_qt) tile(t + 1, 2, Flag<true>{});
      if (t + 2 < n_qt) tile(t + 2, 0, Flag<true>{});
    }
    // The last dV, dK products (tile n_qt - 1, in buffer (n_qt - 1) % 3).
    {
      const int jl = (n_qt - 1) % 3;
      const uint32_t qol = jl == 0 ? qbuf(0) : (jl == 1 ? qbuf(1) : qbuf(2));
      const uint32_t dol = jl == 0 ? dobuf(0) : (jl == 1 ? dobuf(1) : dobuf(2));
      // (dV from dO^T, then dK from Q^T; each operand two reads, issued two products ahead)
      auto rd = [&](int m) __attribute__((always_inline)) {
        const int i = m % NVM;
        return ta.read_tr_rt(m < NVM ? dol : qol, i / NDB, i % NDB);
      };
      constexpr int NL = 2 * NVM;
      bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const bf16x8 a = a0;
        a0 = a1;
        if (m + 2 < NL) a1 = rd(m + 2);
        lds_wait(2 * ((m + 2 < NL ? m + 2 : NL - 1) - m));
        __builtin_amdgcn_sched_barrier(0);
        if (m < NVM) dvacc[m % NDB] = mfma_bf16(a, pb[m / NDB], dvacc[m % NDB]);
        else dkacc[(m - NVM) % NDB] = mfma_bf16(a, dsb[(m - NVM) / NDB], dkacc[(m - NVM) % NDB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (gr == 0) __syncthreads();
  }

  // dK = scale (dK^T)^T, dV: lane column = mykey, register r = dim 32 db + 8 (r/4) + 4 g + r%4.
  // Both leave through the V block's LDS (free once every wave is past its last read),
  // one after the other in the same wave-private slice, so that each store writes whole rows.
  static_assert(8 * 32 * D <= kBwdKeysPP * D, "eight 32-row slices fit in the V block");
  __syncthreads();
  bf16* const slice = sV + wave * (32 * D);
  {
    u32x2 w[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[db][j][0] = pack_bf16x2(dkacc[db][4 * j] * p.scale, dkacc[db][4 * j + 1] * p.scale);
        w[db][j][1] = pack_bf16x2(dkacc[db][4 * j + 2] * p.scale, dkacc[db][4 * j + 3] * p.scale);
      }
    store_rows_via_lds<D>(slice, w, p.dk + base, p.sn, kw0, N, lane);
  }
  __builtin_amdgcn_wave_barrier();
  {
    u32x2 w[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[db][j][0] = pack_bf16x2(dvacc[db][4 * j], dvacc[db][4 * j + 1]);
        w[db][j][1] = pack_bf16x2(dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
      }
    store_rows_via_lds<D>(slice, w, p.dv + base, p.sn, kw0, N, lane);
  }
}

// --------------------------------------------------------------- dQ, two wave groups

// The dQ pass with the products and the element work in different waves at any one
// time (the scheme of the two-group forward): 8 waves own 256 query rows, waves w and
// w + 4 share a SIMD and form two groups that run half a key tile apart, separated by
// workgroup barriers. Wave (group gr, index wg) owns the 32 rows q0 + 64 wg + 32 gr ..
//   product phase t:  dQ^T += K_{t-1}^T dS^T(t - 1), S^T(t) = K_t Q^T, dP^T(t) = V_t dO^T;
//   element phase t:  mask, P = 2^(c S - lse2), dS = P (dP - D), bf16 packing of dS.
// K tiles are kept for three tiles (tile t - 1 is read by the dQ products of phase t),
// V tiles for two; group 0 copies tile t + 1's K and V during its product phase t and
// waits for them at the end of its element phase t (splitting the copies between the
// groups, with V kept for three tiles, measured 1% slower).
constexpr int kBwdRowsPP = 256;
#ifndef FA_BWD_DQ_PP_AHEAD
#define FA_BWD_DQ_PP_AHEAD 3
#endif

template <int D, int BC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_pp_kernel(BwdKParams p) {
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int TILE = BC * D;
  constexpr int NS = NKK * NKB;          // S products (as many dP products)
  constexpr int NQM = (BC / 16) * NDB;   // dQ products
  constexpr int NCP = BC * D / 8 / (64 * 4);  // copies per wave of group 0 per tile (K or V)
  __shared__ __attribute__((aligned(16))) bf16 sT[5 * TILE];  // [K0 | K1 | K2 | V0 | V1]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_wave_id();
  const int gr = wave >> 2, wg = wave & 3;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_blocks, inst, rank);
  const int qb = p.causal ? (p.n_blocks - 1 - rank) : rank;  // heaviest causal rows first
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = p.q + base;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;
  const bf16* dOh = p.dout + base;
  const int q0 = qb * kBwdRowsPP;
  const int wrow0 = q0 + 64 * wg + 32 * gr;
  const int qrow = wrow0 + l32;
  const int qc = min(qrow, N - 1);
  const int64_t rowbase = (int64_t)inst * N;
  int kv_len = N;
  if (p.key_len) kv_len = min(max(p.key_len[b], 0), N);
  int kv_end = kv_len;
  if (p.causal) kv_end = min(kv_end, q0 + kBwdRowsPP);
  const int nt = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // This lane's rows of Q and dO as B operands (dims [16 kk + 8 g, +8)).
  bf16x8 qf[NKK], df[NKK];
  const int64_t qoff = (int64_t)qc * p.sn + 8 * g;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + qoff + 16 * kk);
    df[kk] = *reinterpret_cast<const bf16x8*>(dOh + qoff + 16 * kk);
  }
  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  TileCopy<BC, D, 4> cp;
  cp.init(wg, lane, p.sn);
  TileAddr<D> ta;
  {
    TileOffsets<D> to;
    to.init(lane);
    ta.init(to, lds_address(sT));
  }
  auto kv0_of = [&](int t) { return min(t, nt - 1) * BC; };
  auto kbuf = [](int j) { return 2 * TILE * j; };        // byte offsets in sT
  auto vbuf = [](int j) { return 2 * TILE * (3 + j); };
  if (nt > 0 && gr == 0) {
    cp.issue(sT + kbuf(0) / 2, Kh, p.sn, kv0_of(0), N);
    cp.issue(sT + vbuf(0) / 2, Vh, p.sn, kv0_of(0), N);
  }

  // D = sum_i dO_i O_i (this lane's half of the dims, then its partner's) and
  // lse2 = LSE log2(e) (+inf for a row with no key), formed while the first copies are
  // in flight and written to the workspace for the dK/dV pass.
  float d_half = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.o + base + qoff + 16 * kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) d_half = fmaf((float)ov[i], (float)df[kk][i], d_half);
  }
  const float d_q = pair_sum(d_half);
  const float lse_q = p.lse[rowbase + qc];
  const float lse2_q = (lse_q == kNegInf) ? kPosInf : lse_q * kLog2e;
  if (qrow < N && g == 0) {
    p.delta[rowbase + qrow] = d_q;
    p.lse2[rowbase + qrow] = lse2_q;
  }

  f32x16 sacc[NKB], dpacc[NKB];
  // Every register of a lane's dP^T block belongs to its own query, so each dP chain starts
  // from -D instead of zero and the element phase takes dP - D from the products (one VALU
  // subtraction fewer per pair; measured 1-1.5% off this pass).
  f32x16 neg_d;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_d[r] = -d_q;
  bf16x8 dsb[2 * NKB];

  // Operand ring of the product phases (slot m % (AH + 1) holds product m's operand). A
  // phase's first AH reads are issued at the end of the element phase before it (PRE):
  // they read K_{t-1}, resident since that tile's own products, and arrive while the
  // waves wait at the barrier instead of after it.
  constexpr int AH = FA_BWD_DQ_PP_AHEAD;
  bf16x8 ra[AH + 1];
  // Issues the LDS reads of product m of a phase (buffers kp, kb, vb); returns their number.
  auto fetch_op = [&](int m, int kp, int kb, int vb, auto dq_flag, bool issue) __attribute__((always_inline)) {
    constexpr int NQ = decltype(dq_flag)::value ? NQM : 0;
    const int sl = m % (AH + 1);
    if (m < NQ) {
      if (issue) ra[sl] = ta.read_tr(kp, m / NDB, m % NDB);
      return 2;
    } else if (m < NQ + NS) {
      const int j = m - NQ;
      if (issue) ra[sl] = ta.read_row(kb, j / NKK, j % NKK);
      return 1;
    } else {
      const int j = m - NQ - NS;
      if (issue) ra[sl] = ta.read_row(vb, j / NKK, j % NKK);
      return 1;
    }
  };
  // Product phase: (DQ) dQ^T += K_{t-1}^T dS^T(t - 1) from the K buffer at kp, then
  // S^T(t) and dP^T(t) from the K / V buffers at kb / vb. LDS operands are inline-
  // assembly reads issued AH products ahead and waited for exactly.
  auto products = [&](int kp, int kb, int vb, auto dq_flag, auto pre_flag) __attribute__((always_inline)) {
    constexpr bool DQ = decltype(dq_flag)::value, PRE = decltype(pre_flag)::value;
    constexpr int NQ = DQ ? NQM : 0;
    constexpr int NM = NQ + 2 * NS;
    int ia[AH + 1];
    int nrd = 0;
    auto fetch = [&](int m, bool issue) __attribute__((always_inline)) {
      nrd += fetch_op(m, kp, kb, vb, dq_flag, issue);
      ia[m % (AH + 1)] = nrd - 1;
    };
#pragma unroll
    for (int m = 0; m < AH && m < NM; ++m) fetch(m, !PRE);
    static_for<NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if (m + AH < NM) fetch(m + AH, true);
      lds_wait(nrd - 1 - ia[m % (AH + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 a = ra[m % (AH + 1)];
      if constexpr (m < NQ) {
        dqacc[m % NDB] = mfma_bf16(a, dsb[m / NDB], dqacc[m % NDB]);
      } else if constexpr (m < NQ + NS) {
        constexpr int j = m - NQ;
        sacc[j / NKK] = mfma_bf16(a, qf[j % NKK], j % NKK == 0 ? f32x16{} : sacc[j / NKK]);
      } else {
        constexpr int j = m - NQ - NS;
        dpacc[j / NKK] = mfma_bf16(a, df[j % NKK], j % NKK == 0 ? neg_d : dpacc[j / NKK]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Element phase of the tile at kv0 (register r of key block kb is key
  // kv0 + 32 kb + 8 (r/4) + 4 g + r%4; a key is kept iff key <= min(kv_len - 1, qrow
  // when causal)).
  auto elements = [&](int kv0) __attribute__((always_inline)) {
    if ((kv0 + BC > kv_len) || (p.causal && kv0 + BC - 1 > wrow0)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int lim = min(kv_len - 1, p.causal ? qrow : 0x3FFFFFFF) - kv0 - 32 * kb - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          if (off > lim) sacc[kb][r] = kNegInf;
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pr = fast_exp2(fmaf(sacc[kb][e], p.c, -lse2_q));
        dpacc[kb][e] = pr * dpacc[kb][e];  // dP - D: the chain started from -D
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const f32x16& S = dpacc[kb];
        const int o = 8 * h8;
        dsb[2 * kb + h8] = pack_bf16x8(S[o], S[o + 1], S[o + 2], S[o + 3], S[o + 4], S[o + 5], S[o + 6], S[o + 7]);
      }
    // (keeps the phase's work inside it)
#pragma unroll
    for (int k = 0; k < 2 * NKB; ++k) asm volatile("" : "+v"(dsb[k]));
  };

  // Both groups run product phase t, barrier, element phase t, barrier; group 1 starts
  // one barrier later, group 0 ends with one extra barrier.
  if (nt > 0) {
    if (gr == 0) wait_vmem();
    __syncthreads();
    if (gr == 1) __syncthreads();
    auto tile = [&](int t, int jk, int jv, auto dq_flag) __attribute__((always_inline)) {
      // K_t in buffer jk, V_t in jv; K_{t-1} in (jk + 2) % 3; tile t + 1 goes to
      // K buffer (jk + 1) % 3 (it held K_{t-2}) and V buffer 1 - jv.
      if (gr == 0) {
        cp.issue(sT + kbuf((jk + 1) % 3) / 2, Kh, p.sn, kv0_of(t + 1), N);
        cp.issue(sT + vbuf(1 - jv) / 2, Vh, p.sn, kv0_of(t + 1), N);
      }
      products(kbuf((jk + 2) % 3), kbuf(jk), vbuf(jv), dq_flag, dq_flag);  // (tiles after the first were prefetched)
      __syncthreads();
      elements(kv0_of(t));
      if (t + 1 < nt) {
#pragma unroll
        for (int m = 0; m < AH; ++m) fetch_op(m, kbuf(jk), kbuf((jk + 1) % 3), vbuf(1 - jv), Flag<true>{}, true);
      }
      if (gr == 0) wait_vmem();
      __syncthreads();
    };
    tile(0, 0, 0, Flag<false>{});
    // Tiles 1.. (buffers K: t % 3, V: t % 2; six per trip so that every buffer offset is
    // a constant).
    for (int t = 1; t < nt; t += 6) {
      tile(t, 1, 1, Flag<true>{});
      if (t + 1 < nt) tile(t + 1, 2, 0, Flag<true>{});
      if (t + 2 < nt) tile(t + 2, 0, 1, Flag<true>{});
      if (t + 3 < nt) tile(t + 3, 1, 0, Flag<true>{});
      if (t + 4 < nt) tile(t + 4, 2, 1, Flag<true>{});
      if (t + 5 < nt) tile(t + 5, 0, 0, Flag<true>{});
    }
    // The last dQ products (tile nt - 1, its K in buffer (nt - 1) % 3).
    {
      const int kl = (nt - 1) % 3;
      const uint32_t klast = kl == 0 ? kbuf(0) : (kl == 1 ? kbuf(1) : kbuf(2));
      constexpr int AH = 2;
      bf16x8 a0 = ta.read_tr_rt(klast, 0, 0);
      bf16x8 a1 = ta.read_tr_rt(klast, 1 / NDB, 1 % NDB);
#pragma unroll
      for (int i = 0; i < NQM; ++i) {
        const bf16x8 a = a0;
        a0 = a1;
        if (i + AH < NQM) a1 = ta.read_tr_rt(klast, (i + AH) / NDB, (i + AH) % NDB);
        lds_wait(2 * ((i + AH < NQM ? i + AH : NQM - 1) - i));
        __builtin_amdgcn_sched_barrier(0);
        dqacc[i % NDB] = mfma_bf16(a, dsb[i / NDB], dqacc[i % NDB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (gr == 0) __syncthreads();
  }

  // dQ = scale dQ^T^T: lane = query, register r = dim 32 db + 8 (r/4) + 4 g + r%4; it leaves
  // through the tile buffers (free once every wave is past its last read) so that each store
  // writes whole rows.
  u32x2 w[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[db][j][0] = pack_bf16x2(dqacc[db][4 * j] * p.scale, dqacc[db][4 * j + 1] * p.scale);
      w[db][j][1] = pack_bf16x2(dqacc[db][4 * j + 2] * p.scale, dqacc[db][4 * j + 3] * p.scale);
    }
  static_assert(8 * 32 * D <= 5 * TILE, "eight 32-row slices fit in the tile buffers");
  __syncthreads();
  store_rows_via_lds<D>(sT + wave * (32 * D), w, p.dq + base, p.sn, wrow0, N, lane);
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
  p.delta = a.delta;
  p.lse2 = a.lse2;
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.B = a.B;
  p.H = a.H;
  p.N = a.N;
  p.scale = a.scale;
  // kept positive (see the forward): masked scores (-inf) then always give P = 0
  p.c = fmaxf(a.scale * kLog2e, 1.17549435e-38f);
  p.causal = a.causal;
  p.key_len = a.key_len;
  p.bmask = a.block_mask;
  p.nb = a.nb;
  p.bs = a.block_size;
  p.n_blocks = (a.N + kBwdBlock - 1) / kBwdBlock;
  const bool sparse = a.block_mask != nullptr;
  const bool smask = a.causal || a.key_len != nullptr;
  const bool drop = a.dropout.p8 != 0;
  p.drop = a.dropout;
  const dim3 block(256);

  constexpr int TQ128 = FA_BWD_TILE_Q_D128, TQ64 = FA_BWD_TILE_Q_D64;
  constexpr int TK128 = FA_BWD_TILE_K_D128, TK64 = FA_BWD_TILE_K_D64;
  const dim3 grid((unsigned)(a.B * a.H * p.n_blocks));
  // The dQ pass first: it also writes each row's D and lse2, which the dK/dV
  // pass reads for every query tile it visits.
  // Block-sparse with dropout always takes the element-masked variant (with neither causal
  // nor key_len no tile needs masking).
  timer_begin("fa_bwd_dq", s);
  if (a.d == 128) {
    if (drop && sparse) bwd_dq_kernel<128, FA_BWD_TILE_K_DROP_D128, true, true, true><<<grid, block, 0, s>>>(p);
    else if (drop) bwd_dq_kernel<128, FA_BWD_TILE_K_DROP_D128, false, false, true><<<grid, block, 0, s>>>(p);
    else if (sparse && smask) bwd_dq_kernel<128, TK128, true, true><<<grid, block, 0, s>>>(p);
    else if (sparse) bwd_dq_kernel<128, TK128, true><<<grid, block, 0, s>>>(p);
    else if (FA_BWD_DQ_PINGPONG) {
      BwdKParams pp = p;
      pp.n_blocks = (a.N + kBwdRowsPP - 1) / kBwdRowsPP;
      bwd_dq_pp_kernel<128, 64><<<dim3((unsigned)(a.B * a.H * pp.n_blocks)), dim3(512), 0, s>>>(pp);
    } else bwd_dq_kernel<128, TK128, false><<<grid, block, 0, s>>>(p);
  } else {
    if (drop && sparse) bwd_dq_kernel<64, TK64, true, true, true><<<grid, block, 0, s>>>(p);
    else if (drop) bwd_dq_kernel<64, TK64, false, false, true><<<grid, block, 0, s>>>(p);
    else if (sparse && smask) bwd_dq_kernel<64, TK64, true, true><<<grid, block, 0, s>>>(p);
    else if (sparse) bwd_dq_kernel<64, TK64, true><<<grid, block, 0, s>>>(p);
    else bwd_dq_kernel<64, TK64, false><<<grid, block, 0, s>>>(p);
  }
  timer_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  timer_begin("fa_bwd_dkdv", s);
  if (a.d == 128) {
    if (drop && sparse) bwd_dkdv_kernel<128, TQ128, true, true, true, true><<<grid, block, 0, s>>>(p);
    else if (drop) bwd_dkdv_kernel<128, TQ128, false, true, false, true><<<grid, block, 0, s>>>(p);
    else if (sparse && smask) bwd_dkdv_kernel<128, TQ128, true, true, true><<<grid, block, 0, s>>>(p);
    else if (sparse) bwd_dkdv_kernel<128, TQ128, true, true><<<grid, block, 0, s>>>(p);
    else if (FA_BWD_DKDV_PINGPONG && TQ128 == 32) {
      BwdKParams pp = p;
      pp.n_blocks = (a.N + kBwdKeysPP - 1) / kBwdKeysPP;
      bwd_dkdv_pp_kernel<128, 32><<<dim3((unsigned)(a.B * a.H * pp.n_blocks)), dim3(512), 0, s>>>(pp);
    } else bwd_dkdv_kernel<128, TQ128, false, true><<<grid, block, 0, s>>>(p);
  } else {
    if (drop && sparse) bwd_dkdv_kernel<64, TQ64, true, false, true, true><<<grid, block, 0, s>>>(p);
    else if (drop) bwd_dkdv_kernel<64, TQ64, false, false, false, true><<<grid, block, 0, s>>>(p);
    else if (sparse && smask) bwd_dkdv_kernel<64, TQ64, true, false, true><<<grid, block, 0, s>>>(p);
    else if (sparse) bwd_dkdv_kernel<64, TQ64, true, false><<<grid, block, 0, s>>>(p);
    else bwd_dkdv_kernel<64, TQ64, false, false><<<grid, block, 0, s>>>(p);
  }
  timer_end(s);
  return hipGetLastError();
}

}  // namespace fa
