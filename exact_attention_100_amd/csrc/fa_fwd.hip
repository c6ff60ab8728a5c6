// Fused exact-attention forward for gfx950.
//
// Method: the tiled forward of "FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness" (reading notes (hackmd), §Algorithm › Tiling and
// Kernel Fusion): a workgroup owns a block of query rows, streams the K/V tiles
// through on-chip memory, keeps a running row max m and row sum l, rescales its
// output accumulator whenever m grows, and writes only O and one statistic per
// row, never the N x N score matrix. The result equals the one-shot softmax
// exactly (up to rounding) by the incremental-aggregation property the same
// section states.
//
// gfx950 mapping (our design):
//   * 4 waves x 32 query rows = 128 rows per workgroup; K/V tiles of BC keys
//     arrive by direct global -> LDS copies, double-buffered, row-major in a
//     swizzled layout; the V^T operand of P V comes from the transposing LDS
//     read (ds_read_b64_tr_b16), two per MFMA.
//   * Each wave computes S^T = K Q^T on the 32x32x16 bf16 MFMA, so a lane owns
//     ONE query column and 16 keys of it: row max / row sum are per-lane
//     reductions plus one exchange with lane l^32, the rescale factor is one
//     scalar per lane, and the probabilities already sit in the B-operand layout
//     of O^T += V^T P^T (no register shuffles).
//   * Q stays in VGPRs for the whole key loop; O^T accumulates in f32.
//   * Heaviest causal rows first; all tiles of a head on one XCD.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

struct FwdKParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t sb, sh, sn;
  int B, H, N;
  float c;  // scale * log2(e): scores are kept in the base-2 domain
  int causal;
  const int32_t* key_len;
  const uint8_t* bmask;  // block-sparse: uint8 [nb][nb], row = query block
  int nb;
  int bs;
  int n_qblocks;
  Dropout drop;
};

constexpr int kFwdRows = 128;  // query rows per workgroup (4 waves x 32)
constexpr float kRescaleSlack = 8.f;

// Key range and tile count of one workgroup, shared by the bf16 and f32 kernels.
struct FwdRange {
  int kv_len;    // keys >= kv_len are masked for every row of this instance
  int n_tiles;   // tiles to visit
  const int16_t* blocks;  // sparse: this query block's kept key blocks (LDS)
};

// Sparse: `blocks` / `n_blocks` are the query block's kept key blocks (blocks above
// the diagonal already dropped when causal); key_len and the diagonal blocks mask
// per element.
template <int BC, bool SPARSE>
__device__ __forceinline__ FwdRange fwd_range(const FwdKParams& p, int b, int q0, const int16_t* blocks = nullptr,
                                              int n_blocks = 0) {
  FwdRange r;
  r.kv_len = p.N;
  r.blocks = blocks;
  if (p.key_len) r.kv_len = min(max(p.key_len[b], 0), p.N);
  if (SPARSE) {
    r.n_tiles = n_blocks * (p.bs / BC);
  } else {
    int kv_end = r.kv_len;
    if (p.causal) kv_end = min(kv_end, q0 + kFwdRows);
    r.n_tiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  }
  return r;
}

template <int BC, bool SPARSE>
__device__ __forceinline__ int fwd_tile_kv0(const FwdKParams& p, const FwdRange& r, int t) {
  if (SPARSE) {
    if (t >= r.n_tiles) return 0;  // (the prologue of an empty row list)
    const int tpb = p.bs / BC;
    const int blk = r.blocks[t / tpb];
    return blk * p.bs + (t - (t / tpb) * tpb) * BC;
  }
  return t * BC;
}

// Masks the S^T registers of a tile (NKB blocks of 32 keys; lane = one query,
// register r of block kb = key kv0 + 32 kb + 8 (r/4) + 4 g + r%4): entries whose
// key is past kv_len or, when causal, after the query become -inf.
template <int NKB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NKB], int kv0, int kv_len, int causal, int qrow, int g) {
  // Register r of block kb is key kv0 + 4 g + off with off = 32 kb + 8 (r/4) + r%4 a
  // compile-time constant, kept iff key <= min(kv_len - 1, qrow when causal): one
  // compare against a constant per entry.
  const int lim = min(kv_len - 1, causal ? qrow : 0x3FFFFFFF) - kv0 - 4 * g;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
      if (off > lim) s[kb][r] = kNegInf;
    }
}

// One online-softmax step over the (masked) S^T registers of a tile. On return
// s[] holds the unnormalised probabilities 2^(c S - m) (exactly 0 where S = -inf,
// as c > 0) and the result is the factor that rescales everything accumulated
// before this tile. The reference point m only moves when the row max exceeds
// it by more than kRescaleSlack (base 2): softmax is invariant to the shift,
// the unnormalised probabilities stay <= 2^kRescaleSlack, and most tiles then
// need no rescale at all.
template <int NKB>
__device__ __forceinline__ float online_softmax_step(f32x16 (&s)[NKB], float c, float& m_run, float& l_run) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx);
  const float mxs = (mx == kNegInf) ? kNegInf : mx * c;
  const float m_new = (mxs > m_run + kRescaleSlack) ? mxs : m_run;
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(m_run - m_use);
  m_run = m_new;
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = fast_exp2(fmaf(s[kb][r], c, -m_use));
      s[kb][r] = pv;
      rs += pv;
    }
  l_run = l_run * alpha + rs;
  return alpha;
}

// ----------------------------------------------------------------------------------- bf16

__device__ __forceinline__ float sum4(const float (&acc)[4]) { return (acc[0] + acc[1]) + (acc[2] + acc[3]); }

// O's normaliser, the row sum of the bf16-rounded probabilities, on the matrix cores:
// one 16x16x32 product per packed P^T operand pb (lane l: 8 probabilities of query
// l % 32). That product reads lane l's 8 values as k-slots 8 (l / 16) .. + 7 of column
// l % 16, so a column's slots come from lanes n, n + 32 (query n) and n + 16, n + 48
// (query n + 16). The A operand below (rowsum_selector) is 1 in rows i whose i / 4 has
// the parity of the slot group and 0 elsewhere: output rows 4 (l / 16) .. + 3 of column
// l % 16, the four registers lane l receives, then all hold the sum of the operand's 16
// probabilities of lane l's own query. Each product replaces 4 v_dot2 (the VALU
// instruction that slows most beside another wave's products) with 16 matrix-core cycles.
__device__ __forceinline__ bf16x8 rowsum_selector(int lane) {
  const bf16 v = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1)) ? (bf16)1.f : (bf16)0.f;
  bf16x8 a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = v;
  return a;
}
__device__ __forceinline__ f32x4 rowsum_mfma(bf16x8 sel, bf16x8 pb, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb, acc, 0, 0, 0);
}

// The bf16 kernels' softmax step: as online_softmax_step, but the probabilities
// are packed to bf16 (pb, the B operands of the P V product; k-step ks = 2 kb + s
// holds registers 8 s .. 8 s + 7 of block kb) and two row sums are kept. O's
// normaliser adds up the rounded values (rowsum_mfma over pb, by the caller): it is
// then the sum of exactly the weights the product applies, so O is a convex
// combination of V rows and a bf16 rounding of a dominant probability cancels
// instead of scaling O. lu_run adds up the unrounded float32 values, the row sum of
// exp(S - m) that LSE = m + ln l is defined with (the running sum of the tiled softmax).
template <int NKB>
__device__ __forceinline__ float softmax_tile_bf16(f32x16 (&s)[NKB], float c, float& m_run, float& lu_run,
                                                   bf16x8 (&pb)[2 * NKB]) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx);
  const float mxs = (mx == kNegInf) ? kNegInf : mx * c;
  const float m_new = (mxs > m_run + kRescaleSlack) ? mxs : m_run;
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(m_run - m_use);
  m_run = m_new;
  float ru[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
      for (int i = 8 * sh; i < 8 * sh + 8; ++i) {
        s[kb][i] = fast_exp2(fmaf(s[kb][i], c, -m_use));
        ru[i & 3] = (kb == 0 && i < 4) ? s[kb][i] : ru[i & 3] + s[kb][i];  // (0 + x = x for x >= 0)
      }
      pb[2 * kb + sh] = pack_bf16x8(s[kb][8 * sh + 0], s[kb][8 * sh + 1], s[kb][8 * sh + 2], s[kb][8 * sh + 3],
                                    s[kb][8 * sh + 4], s[kb][8 * sh + 5], s[kb][8 * sh + 6], s[kb][8 * sh + 7]);
    }
  lu_run = lu_run * alpha + sum4(ru);
  return alpha;
}

// Waves per SIMD the bf16 forward is compiled for: two, so that one wave's
// softmax (VALU, transcendental) overlaps the other wave's MFMA work.
#ifndef FA_FWD_WAVES_PER_EU
#define FA_FWD_WAVES_PER_EU 2
#endif

// SMASK: a block-sparse launch that also applies the causal / key-length
// element masks (without it, sparse tiles are never masked). DROP: dropout on P
// (dense and block-sparse launches): dropped entries of the packed bf16
// probabilities are zeroed after both row sums have taken them, and O is scaled by
// 1 / (1 - p) at the end.
template <int D, int BC, bool SPARSE, bool SMASK = false, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FA_FWD_WAVES_PER_EU)))
void fwd_bf16_kernel(FwdKParams p) {
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int TILE = BC * D;

  // K and V tiles, double-buffered, row-major in the swizzled layout (16-byte
  // row reads for the K operand, transposing reads for the V^T operand), in one
  // array [K0 | K1 | V0 | V1]. Every read is inline assembly: each lane's
  // addresses are computed once and a read names its buffer by the instruction's
  // immediate offset (the key loop is unrolled by two, so those fold).
  __shared__ __attribute__((aligned(16))) bf16 sT[4 * TILE];
  bf16* const sK0 = sT;
  bf16* const sK1 = sT + TILE;
  bf16* const sV0 = sT + 2 * TILE;
  bf16* const sV1 = sT + 3 * TILE;
  // Block-sparse: this query block's kept key blocks.
  __shared__ int16_t sBlk[SPARSE ? kMaxBlocks : 1];
  __shared__ int sBlkN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_qblocks, inst, rank);
  const int qb = (!SPARSE && p.causal) ? (p.n_qblocks - 1 - rank) : rank;
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = static_cast<const bf16*>(p.q) + base;
  const bf16* Kh = static_cast<const bf16*>(p.k) + base;
  const bf16* Vh = static_cast<const bf16*>(p.v) + base;
  const int q0 = qb * kFwdRows;
  const int qrow = q0 + wave * 32 + l32;
  int n_blk = 0;
  if constexpr (SPARSE) n_blk = kept_block_list<true>(p.bmask, p.nb, q0 / p.bs, p.causal, sBlk, &sBlkN);
  const FwdRange rg = fwd_range<BC, SPARSE>(p, b, q0, sBlk, n_blk);

  // Every global load is unconditional: rows past the end are clamped to row
  // N - 1, whose values then only ever meet probability 0 (masked keys) or feed
  // outputs that are not stored (query rows >= N).
  // This lane's query, as the B operand of S^T = K Q^T: slot group g of k-step
  // kk holds dims [16 kk + 8 g, 16 kk + 8 g + 8).
  bf16x8 qf[NKK];
  const int64_t qoff = (int64_t)min(qrow, N - 1) * p.sn;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + qoff + 16 * kk + 8 * g);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, lu_run = 0.f;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};  // O's normaliser (rowsum_mfma; every register holds it)
  const bf16x8 sel = rowsum_selector(lane);

  // Software pipeline over the key tiles. Iteration t computes S(t) = K_t Q^T,
  // then the P V product of tile t - 1 interleaved with the softmax of tile t, so
  // that the softmax's VALU and exp work runs while the MFMA pipe executes
  // P_{t-1} V_{t-1}. The V tile therefore trails the K tile by one: iteration t
  // copies K_{t+1} and V_t (direct global -> LDS copies, two buffers each; the
  // last iterations re-read the last tile so that memory operations are never
  // predicated).
  TileCopy<BC, D, 4> cp;
  cp.init(uniform_wave_id(), lane, p.sn);
  TileAddr<D> ta;
  {
    TileOffsets<D> to;
    to.init(lane);
    ta.init(to, lds_address(sT));
  }
  const int nt = rg.n_tiles;
  auto kv0_of = [&](int t) { return fwd_tile_kv0<BC, SPARSE>(p, rg, min(t, nt - 1)); };

  // S^T (keys x queries) = K_tile Q^T. MFMA j is k-step j / NKB of key block j % NKB.
  // The K operands are inline-assembly LDS reads kAhead MFMAs ahead of their
  // use, each waited for exactly (lds_wait): with copies in flight the compiler
  // would drain every LDS read before each product.
  auto s_mfma = [&](const bf16* sk, f32x16 (&sacc)[NKB]) __attribute__((always_inline)) {
    constexpr int NS = NKK * NKB, kAhead = 4;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    const int off = (int)(lds_address(sk) - lds_address(sT));
    bf16x8 ring[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) ring[j] = ta.read_row(off, j % NKB, j / NKB);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bf16x8 a = ring[j % kAhead];
      if (j + kAhead < NS) ring[j % kAhead] = ta.read_row(off, (j + kAhead) % NKB, (j + kAhead) / NKB);
      lds_wait(NS - 1 - j < kAhead ? NS - 1 - j : kAhead);  // the reads issued after operand j
      __builtin_amdgcn_sched_barrier(0);
      sacc[j % NKB] = mfma_bf16(a, qf[j / NKB], sacc[j % NKB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T (dims x queries) += V^T P^T; A = V^T through the transposing LDS read,
  // whose key slots are the same as those of pb.
  auto pv_mfma = [&](const bf16* sv, const bf16x8 (&pb)[2 * NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = ta.read_tr((int)(lds_address(sv) - lds_address(sT)), ks, db);
        lds_wait(0);
        // (the wait does not order the product by itself: nothing it touches is an operand)
        __builtin_amdgcn_sched_barrier(0);
        oacc[db] = mfma_bf16(a, pb[ks], oacc[db]);
      }
  };
  // Dropout of one tile's packed probabilities (k-step ks = 2 kb + s holds the key
  // quads 32 kb + 16 s + 4 g and that + 8 of this lane's query).
  // (Quad c = 4 kb + 2 s + h is keys kv0 + 4 g + 8 c .. + 3.)
  auto drop_tile = [&](bf16x8 (&pk)[2 * NKB], int kv0) __attribute__((always_inline)) {
    uint32_t w[4 * NKB];
    dropout_row_words<4 * NKB>(p.drop, qrow, kv0 + 4 * g, (uint32_t)inst, w);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        pk[2 * kb + s] = dropout_apply8(pk[2 * kb + s], w[4 * kb + 2 * s], w[4 * kb + 2 * s + 1], p.drop.p8);
  };
  auto needs_mask = [&](int kv0) {
    return (!SPARSE || SMASK) && ((kv0 + BC > rg.kv_len) || (p.causal && kv0 + BC - 1 > q0 + wave * 32));
  };

  if (nt > 0) {
    bf16x8 pb[2 * NKB];
    cp.issue(sK0, Kh, p.sn, kv0_of(0), N);
    wait_vmem();
    __syncthreads();
    cp.issue(sK1, Kh, p.sn, kv0_of(1), N);
    cp.issue(sV0, Vh, p.sn, kv0_of(0), N);
    {
      f32x16 sacc[NKB];
      s_mfma(sK0, sacc);
      if (needs_mask(kv0_of(0))) mask_tile<NKB>(sacc, kv0_of(0), rg.kv_len, p.causal, qrow, g);
      // P^T as B operands: k-step ks = 2 kb + s covers keys 32 kb + 16 s +
      // {4g..4g+3, 8+4g..8+4g+3}. (alpha is irrelevant: nothing accumulated yet.)
      softmax_tile_bf16<NKB>(sacc, p.c, m_run, lu_run, pb);
#pragma unroll
      for (int k = 0; k < 2 * NKB; ++k) lacc = rowsum_mfma(sel, pb[k], lacc);
      if (DROP) drop_tile(pb, kv0_of(0));
    }
    wait_vmem();
    __syncthreads();

    // Iteration t: K_{t+1} -> kw, V_t -> vw, S(t) from kr, P V of tile t - 1 from vr.
    auto iteration = [&](int t, bf16* kw, const bf16* kr, bf16* vw, const bf16* vr) __attribute__((always_inline)) {
      const int kv0 = kv0_of(t);
      cp.issue(kw, Kh, p.sn, kv0_of(t + 1), N);
      cp.issue(vw, Vh, p.sn, kv0, N);
      f32x16 sacc[NKB];
      s_mfma(kr, sacc);
      if (needs_mask(kv0)) mask_tile<NKB>(sacc, kv0, rg.kv_len, p.causal, qrow, g);

      // The P V of tile t - 1 and the softmax of tile t are independent. They are
      // interleaved by hand, one slice of softmax work per P V MFMA (scheduling
      // fences keep the slices in place): slices 0-1 the row max, slice 2 the new
      // reference point, the rest the exponentials, the unrounded row sum and bf16
      // packing; O's normaliser follows as rowsum_mfma products after the slices.
      // The transposing LDS reads of each MFMA's operand run two slices ahead.
      constexpr int NPV = NDB * (BC / 16);
      constexpr int NE = NKB * 16;  // scores per lane
      constexpr int NEXP = NPV - 3; // slices doing exponentials
      static_assert(NPV >= 4, "too few MFMAs to interleave");
      bf16x8 pbn[2 * NKB];
      const int voff = (int)(lds_address(vr) - lds_address(sT));
      bf16x8 a0 = ta.read_tr(voff, 0, 0);
      bf16x8 a1 = ta.read_tr(voff, 1 / NDB, 1 % NDB);
      // (row max as four running maxima, each slice extending all four: independent
      // v_max3 chains instead of one dependent chain per slice)
      float t4[4] = {kNegInf, kNegInf, kNegInf, kNegInf}, m_new = 0.f, m_use = 0.f, alpha = 1.f;
      float rup[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const bf16x8 a = a0;
        a0 = a1;
        if (i + 2 < NPV) a1 = ta.read_tr(voff, (i + 2) / NDB, (i + 2) % NDB);
        lds_wait(2 * ((i + 2 < NPV ? i + 2 : NPV - 1) - i));  // two reads per later operand
        __builtin_amdgcn_sched_barrier(0);
        oacc[i % NDB] = mfma_bf16(a, pb[i / NDB], oacc[i % NDB]);
        if (i == 0) {
#pragma unroll
          for (int e = 0; e < NE / 2; ++e) t4[(e / 4) & 3] = fmaxf(t4[(e / 4) & 3], sacc[e / 16][e % 16]);
        } else if (i == 1) {
#pragma unroll
          for (int e = NE / 2; e < NE; ++e) t4[(e / 4) & 3] = fmaxf(t4[(e / 4) & 3], sacc[e / 16][e % 16]);
        } else if (i == 2) {
          const float mx = pair_max(fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3])));
          const float mxs = (mx == kNegInf) ? kNegInf : mx * p.c;
          m_new = (mxs > m_run + kRescaleSlack) ? mxs : m_run;
          m_use = (m_new == kNegInf) ? 0.f : m_new;
          alpha = fast_exp2(m_run - m_use);
        } else {
          const int s0 = ((i - 3) * NE) / NEXP, s1 = ((i - 2) * NE) / NEXP;
#pragma unroll
          for (int e = s0; e < s1; ++e) {
            sacc[e / 16][e % 16] = fast_exp2(fmaf(sacc[e / 16][e % 16], p.c, -m_use));
            rup[e & 3] = e < 4 ? sacc[e / 16][e % 16] : rup[e & 3] + sacc[e / 16][e % 16];
            if ((e & 7) == 7) {  // a group of 8 probabilities is complete: pack it
              const int kb = e / 16, s8 = (e % 16) / 8;
              pbn[2 * kb + s8] = pack_bf16x8(sacc[kb][8 * s8 + 0], sacc[kb][8 * s8 + 1], sacc[kb][8 * s8 + 2],
                                             sacc[kb][8 * s8 + 3], sacc[kb][8 * s8 + 4], sacc[kb][8 * s8 + 5],
                                             sacc[kb][8 * s8 + 6], sacc[kb][8 * s8 + 7]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Consume the slice results here so that no later pass sinks them past the
      // rescale branch, out of the slices they were placed in.
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) asm volatile("" : "+v"(pbn[i]));
      float ru = sum4(rup);
      asm volatile("" : "+v"(ru), "+v"(alpha), "+v"(m_new));
      const float m_prev = m_run;
      m_run = m_new;
      lu_run = lu_run * alpha + ru;
      // alpha == 1 exactly when no row of this wave moved its reference max.
      if (__builtin_amdgcn_ballot_w64(m_run != m_prev)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        lacc *= alpha;
      }
      // O's normaliser takes this tile's rounded probabilities before dropout.
#pragma unroll
      for (int k = 0; k < 2 * NKB; ++k) lacc = rowsum_mfma(sel, pbn[k], lacc);
      if (DROP) drop_tile(pbn, kv0);
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) pb[i] = pbn[i];
      wait_vmem();
      __syncthreads();
    };
    for (int t = 1; t < nt; t += 2) {
      iteration(t, sK0, sK1, sV1, sV0);
      if (t + 1 < nt) iteration(t + 1, sK1, sK0, sV0, sV1);
    }
    // The last tile's V is in sV1 when nt is even, in sV0 when nt is odd.
    if (nt & 1) pv_mfma(sV0, pb);
    else pv_mfma(sV1, pb);
  }

  // Epilogue: O = O_acc / l (the rounded weights' sum), LSE = (m + log2 lu) ln 2 (the
  // unrounded sum). Rows with no key: O = 0, LSE = -inf.
  const float l_tot = lacc[0];
  const float lu_tot = pair_sum(lu_run);
  const float inv = l_tot > 0.f ? (DROP ? p.drop.scale : 1.f) / l_tot : 0.f;
  // O leaves through the tile buffers (free once every wave is past its last read) so that
  // each store writes whole rows.
  u32x2 w[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[db][j][0] = pack_bf16x2(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
      w[db][j][1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
    }
  static_assert(4 * 32 * D <= 4 * TILE, "four 32-row slices fit in the tile buffers");
  __syncthreads();
  store_rows_via_lds<D>(sT + uniform_wave_id() * (32 * D), w, static_cast<bf16*>(p.o) + base, p.sn, q0 + 32 * wave,
                        N, lane);
  if (qrow < N && g == 0)
    p.lse[(int64_t)inst * N + qrow] = lu_tot > 0.f ? (m_run + fast_log2(lu_tot)) * kLn2 : kNegInf;
}

// -------------------------------------------------------------------- bf16, two wave groups

// The forward with the products and the softmax in different waves at any one time.
// A workgroup of 8 waves owns 256 query rows: waves w and w + 4 share a SIMD and form
// two groups (w < 4 and w >= 4) that run half a key tile apart. In one phase group 0
// issues the products of tile t (S(t) = K_t Q^T, then the P V of tile t - 1) while
// group 1 runs the softmax of tile t - 1; in the next phase the roles swap (workgroup
// barriers separate the phases). A wave that only issues products (and their operand
// reads) keeps the matrix core busy while the wave beside it on the SIMD issues its
// VALU work, so each SIMD overlaps the two kinds of work instead of interleaving them
// inside one instruction stream. The arithmetic is that of fwd_bf16_kernel in the same
// order (same products per accumulator, the normaliser's products after each tile's
// rescale, the same unrounded row-sum chains), so the two kernels give the same bits.
// Wave (group gr, index wg) owns the 32 rows q0 + 64 wg + 32 gr ..: the two waves of a
// SIMD see the same key tiles, and both groups visit the same tiles of the diagonal.
// K/V tiles are double-buffered and copied by group 0 at the start of its product
// phases: phase t issues tile t + 1's K and tile t's V, waited for at the end of
// group 0's softmax phase t.
constexpr int kFwdRowsPP = 256;
#ifndef FA_FWD_PP_AHEAD
#define FA_FWD_PP_AHEAD 4
#endif

template <int D, int BC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_pp_kernel(FwdKParams p) {
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  constexpr int TILE = BC * D;
  constexpr int NS = NKK * NKB;          // S products per tile
  constexpr int NPV = NDB * (BC / 16);   // P V products per tile
  constexpr int NE = NKB * 16;           // scores per lane and tile
  __shared__ __attribute__((aligned(16))) bf16 sT[4 * TILE];  // [K0 | K1 | V0 | V1]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_wave_id();
  const int gr = wave >> 2, wg = wave & 3;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_qblocks, inst, rank);
  const int qb = p.causal ? (p.n_qblocks - 1 - rank) : rank;
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bf16* Qh = static_cast<const bf16*>(p.q) + base;
  const bf16* Kh = static_cast<const bf16*>(p.k) + base;
  const bf16* Vh = static_cast<const bf16*>(p.v) + base;
  const int q0 = qb * kFwdRowsPP;
  const int wrow0 = q0 + 64 * wg + 32 * gr;  // this wave's first row
  const int qrow = wrow0 + l32;
  int kv_len = N;
  if (p.key_len) kv_len = min(max(p.key_len[b], 0), N);
  int kv_end = kv_len;
  if (p.causal) kv_end = min(kv_end, q0 + kFwdRowsPP);
  const int nt = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // This lane's query (B operand of S^T = K Q^T; slot group g of k-step kk holds
  // dims [16 kk + 8 g, +8)); rows past N are clamped and never stored.
  bf16x8 qf[NKK];
  const int64_t qoff = (int64_t)min(qrow, N - 1) * p.sn;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + qoff + 16 * kk + 8 * g);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, lu_run = 0.f;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};  // O's normaliser (rowsum_mfma; every register holds it)
  const bf16x8 sel = rowsum_selector(lane);
  f32x16 sacc[NKB];
  bf16x8 pb[2 * NKB];

  TileCopy<BC, D, 4> cp;
  cp.init(wg, lane, p.sn);
  TileAddr<D> ta;
  {
    TileOffsets<D> to;
    to.init(lane);
    ta.init(to, lds_address(sT));
  }
  auto kv0_of = [&](int t) { return min(t, nt - 1) * BC; };
  constexpr int KB0 = 0, KB1 = 2 * TILE, VB0 = 4 * TILE, VB1 = 6 * TILE;  // byte offsets in sT

  // Product phase: S(t) from the K buffer at byte offset kb, then (PV) the P V product
  // of the previous tile from the V buffer at vb. Every LDS operand is an inline-assembly
  // read issued AH products ahead and waited for exactly (reads return in order).
  auto products = [&](int kb, int vb, auto pv_flag) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_flag)::value;
    constexpr int NM = NS + (PV ? NPV : 0), AH = FA_FWD_PP_AHEAD;
    bf16x8 ra[AH + 1];
    int ia[AH + 1];
    int nrd = 0;
    auto fetch = [&](int m) __attribute__((always_inline)) {
      const int sl = m % (AH + 1);
      if (m < NS) {
        ra[sl] = ta.read_row(kb, m % NKB, m / NKB);
        nrd += 1;
      } else {
        const int i = m - NS;
        ra[sl] = ta.read_tr(vb, i / NDB, i % NDB);
        nrd += 2;
      }
      ia[sl] = nrd - 1;
    };
#pragma unroll
    for (int m = 0; m < AH && m < NM; ++m) fetch(m);
    static_for<NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if (m + AH < NM) fetch(m + AH);
      lds_wait(nrd - 1 - ia[m % (AH + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 a = ra[m % (AH + 1)];
      if constexpr (m < NS) {
        sacc[m % NKB] = mfma_bf16(a, qf[m / NKB], m < NKB ? f32x16{} : sacc[m % NKB]);
      } else {
        constexpr int i = m - NS;
        oacc[i % NDB] = mfma_bf16(a, pb[i / NDB], oacc[i % NDB]);
        if constexpr (i % NDB == NDB - 1) lacc = rowsum_mfma(sel, pb[i / NDB], lacc);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Softmax phase of the tile at kv0: mask (only where the tile needs it), row max,
  // reference point, exponentials, the unrounded row sum (four partial sums, combined as
  // in fwd_bf16_kernel), bf16 packing into pb, and the rescale of O and of its normaliser
  // when a row's reference point moved (the normaliser's products for pb run beside the
  // P V products of the next product phase).
  auto softmax = [&](int kv0) __attribute__((always_inline)) {
    if ((kv0 + BC > kv_len) || (p.causal && kv0 + BC - 1 > wrow0)) mask_tile<NKB>(sacc, kv0, kv_len, p.causal, qrow, g);
    // (four running maxima: chains the compiler turns into v_max3 without
    // canonicalising every score first, as it does for a pairwise tree)
    float t4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int e = 0; e < NE; ++e) t4[(e / 8) & 3] = fmaxf(t4[(e / 8) & 3], sacc[e / 16][e % 16]);
    const float mx = pair_max(fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3])));
    const float mxs = (mx == kNegInf) ? kNegInf : mx * p.c;
    const float m_new = (mxs > m_run + kRescaleSlack) ? mxs : m_run;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float ru[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      sacc[e / 16][e % 16] = fast_exp2(fmaf(sacc[e / 16][e % 16], p.c, -m_use));
      ru[e & 3] = e < 4 ? sacc[e / 16][e % 16] : ru[e & 3] + sacc[e / 16][e % 16];  // (0 + x = x for x >= 0)
    }
#pragma unroll
    for (int k = 0; k < 2 * NKB; ++k) {
      const int kb = k / 2, s8 = 8 * (k % 2);
      pb[k] = pack_bf16x8(sacc[kb][s8 + 0], sacc[kb][s8 + 1], sacc[kb][s8 + 2], sacc[kb][s8 + 3], sacc[kb][s8 + 4],
                          sacc[kb][s8 + 5], sacc[kb][s8 + 6], sacc[kb][s8 + 7]);
    }
    const float m_prev = m_run;
    m_run = m_new;
    lu_run = lu_run * alpha + sum4(ru);
    if (__builtin_amdgcn_ballot_w64(m_run != m_prev)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      lacc *= alpha;
    }
    // (keeps the phase's work inside it: nothing may sink past the barrier's wait)
#pragma unroll
    for (int k = 0; k < 2 * NKB; ++k) asm volatile("" : "+v"(pb[k]));
    asm volatile("" : "+v"(lu_run));
  };

  // Both groups run the same sequence (product phase t, barrier, softmax phase t,
  // barrier); group 1 starts one barrier later, which puts each group's products beside
  // the other group's softmax. Group 0 ends with one extra barrier so that both groups
  // meet the same number.
  if (nt > 0) {
    if (gr == 0) {
      cp.issue(sT + KB0 / 2, Kh, p.sn, kv0_of(0), N);
      wait_vmem();
    }
    __syncthreads();
    if (gr == 1) __syncthreads();
    // Tile 0 (no P V yet).
    if (gr == 0) {
      cp.issue(sT + KB1 / 2, Kh, p.sn, kv0_of(1), N);
      cp.issue(sT + VB0 / 2, Vh, p.sn, kv0_of(0), N);
    }
    products(KB0, VB1, Flag<false>{});
    __syncthreads();
    softmax(kv0_of(0));
    if (gr == 0) wait_vmem();
    __syncthreads();
    // Tile t >= 1: K_t in kb, V_{t-1} in vbp; group 0 copies K_{t+1} into kbn and V_t
    // into vb (two per trip so that every buffer offset is a constant).
    auto tile = [&](int t, int kb, int kbn, int vb, int vbp) __attribute__((always_inline)) {
      if (gr == 0) {
        cp.issue(sT + kbn / 2, Kh, p.sn, kv0_of(t + 1), N);
        cp.issue(sT + vb / 2, Vh, p.sn, kv0_of(t), N);
      }
      products(kb, vbp, Flag<true>{});
      __syncthreads();
      softmax(kv0_of(t));
      if (gr == 0) wait_vmem();
      __syncthreads();
    };
    for (int t = 1; t < nt; t += 2) {
      tile(t, KB1, KB0, VB1, VB0);
      if (t + 1 < nt) tile(t + 1, KB0, KB1, VB0, VB1);
    }
    // The last P V (tile nt - 1, its V in buffer (nt - 1) % 2).
    const uint32_t vlast = ((nt - 1) & 1) ? VB1 : VB0;
    auto read_last = [&](int ks, int db) __attribute__((always_inline)) { return ta.read_tr_rt(vlast, ks, db); };
    {
      constexpr int AH = 2;
      bf16x8 a0 = read_last(0, 0);
      bf16x8 a1 = read_last(1 / NDB, 1 % NDB);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const bf16x8 a = a0;
        a0 = a1;
        if (i + AH < NPV) a1 = read_last((i + AH) / NDB, (i + AH) % NDB);
        lds_wait(2 * ((i + AH < NPV ? i + AH : NPV - 1) - i));
        __builtin_amdgcn_sched_barrier(0);
        oacc[i % NDB] = mfma_bf16(a, pb[i / NDB], oacc[i % NDB]);
        if (i % NDB == NDB - 1) lacc = rowsum_mfma(sel, pb[i / NDB], lacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (gr == 0) __syncthreads();
  }

  // Epilogue: O = O_acc / l (the rounded weights' sum), LSE = (m + log2 lu) ln 2. O goes
  // out through the tile buffers, free once every wave is past its last read of them.
  const float l_tot = lacc[0];
  const float lu_tot = pair_sum(lu_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  u32x2 w[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[db][j][0] = pack_bf16x2(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
      w[db][j][1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
    }
  static_assert(8 * 32 * D <= 4 * TILE, "eight 32-row slices fit in the tile buffers");
  __syncthreads();
  store_rows_via_lds<D>(sT + wave * (32 * D), w, static_cast<bf16*>(p.o) + base, p.sn, wrow0, N, lane);
  if (qrow < N && g == 0)
    p.lse[(int64_t)inst * N + qrow] = lu_tot > 0.f ? (m_run + fast_log2(lu_tot)) * kLn2 : kNegInf;
}

// ------------------------------------------------------------------------------------ f32

// Same schedule and softmax; products on the 32x32x2 f32 MFMA (K index = lane group),
// so both K and V stay row-major in LDS.
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdKParams p) {
  constexpr int BC = 32;
  constexpr int KP = D + 4;  // 16-byte rows
  constexpr int VP = D + 8;  // lane groups (keys 4 apart) land on different banks
  constexpr int NDB = D / 32;
  constexpr int CHUNKS = BC * D / 4 / 256;  // 16-byte chunks per thread per tile (K and V each)
  static_assert(CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) float sK[2][BC * KP];
  __shared__ __attribute__((aligned(16))) float sV[2][BC * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int N = p.N;
  int inst, rank;
  schedule_tile(blockIdx.x, p.B * p.H, p.n_qblocks, inst, rank);
  const int qb = p.causal ? (p.n_qblocks - 1 - rank) : rank;
  const int b = inst / p.H, h = inst - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const float* Qh = static_cast<const float*>(p.q) + base;
  const float* Kh = static_cast<const float*>(p.k) + base;
  const float* Vh = static_cast<const float*>(p.v) + base;
  const int q0 = qb * kFwdRows;
  const int qrow = q0 + wave * 32 + l32;
  const FwdRange rg = fwd_range<BC, false>(p, b, q0);

  float qf[D / 2];  // k-step kk: dim 2 kk + g
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = (qrow < N) ? Qh[(int64_t)qrow * p.sn + 2 * kk + g] : 0.f;

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 kreg[CHUNKS], vreg[CHUNKS];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int ci = tid + 256 * i, r = ci / (D / 4), cc = ci - r * (D / 4);
      const int key = kv0 + r;
      kreg[i] = key < N ? *reinterpret_cast<const f32x4*>(Kh + (int64_t)key * p.sn + 4 * cc) : zero4;
      vreg[i] = key < N ? *reinterpret_cast<const f32x4*>(Vh + (int64_t)key * p.sn + 4 * cc) : zero4;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int ci = tid + 256 * i, r = ci / (D / 4), cc = ci - r * (D / 4);
      *reinterpret_cast<f32x4*>(&sK[buf][r * KP + 4 * cc]) = kreg[i];
      *reinterpret_cast<f32x4*>(&sV[buf][r * VP + 4 * cc]) = vreg[i];
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  if (rg.n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < rg.n_tiles; ++t) {
    const int buf = t & 1;
    const int kv0 = t * BC;
    if (t + 1 < rg.n_tiles) load_tile(kv0 + BC);

    f32x16 sacc[1];
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[0][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) sacc[0] = mfma_f32(sK[buf][l32 * KP + 2 * kk + g], qf[kk], sacc[0]);

    const bool need_mask = (kv0 + BC > rg.kv_len) || (p.causal && kv0 + BC - 1 > q0 + wave * 32);
    if (need_mask) mask_tile<1>(sacc, kv0, rg.kv_len, p.causal, qrow, g);
    const float alpha = online_softmax_step<1>(sacc, p.c, m_run, l_run);
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T: k-step r uses key 8 (r/4) + 4 g + r%4 in lane group g.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma_f32(sV[buf][key * VP + db * 32 + l32], sacc[0][r], oacc[db]);
    }

    if (t + 1 < rg.n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    float* Orow = static_cast<float*>(p.o) + base + (int64_t)qrow * p.sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 w;
        w[0] = oacc[db][4 * j + 0] * inv;
        w[1] = oacc[db][4 * j + 1] * inv;
        w[2] = oacc[db][4 * j + 2] * inv;
        w[3] = oacc[db][4 * j + 3] * inv;
        *reinterpret_cast<f32x4*>(Orow + db * 32 + 8 * j + 4 * g) = w;
      }
    if (g == 0)
      p.lse[(int64_t)inst * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

// ------------------------------------------------------------------------------ launchers

static FwdKParams make_params(const FwdArgs& a) {
  FwdKParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.B = a.B;
  p.H = a.H;
  p.N = a.N;
  // scale * log2(e), kept positive: with scale = 0 the smallest normal float makes
  // every 2^(c S - m) round to exactly 1 (uniform weights, as for c = 0) while
  // masked scores (-inf) still give exactly 0.
  p.c = fmaxf(a.scale * kLog2e, 1.17549435e-38f);
  p.causal = a.causal;
  p.key_len = a.key_len;
  p.bmask = a.block_mask;
  p.nb = a.nb;
  p.bs = a.block_size;
  p.n_qblocks = (a.N + kFwdRows - 1) / kFwdRows;
  p.drop = a.dropout;
  return p;
}

// Keys per K/V tile of the bf16 forward, per head dim.
#ifndef FA_FWD_BC_D128
#define FA_FWD_BC_D128 64
#endif
#ifndef FA_FWD_BC_D64
#define FA_FWD_BC_D64 64
#endif
// Dense d = 128 (no dropout): the two-group kernel and its key tile.
#ifndef FA_FWD_PINGPONG
#define FA_FWD_PINGPONG 1
#endif
#ifndef FA_FWD_PP_BC
#define FA_FWD_PP_BC 64
#endif
#ifndef FA_FWD_PP_AHEAD
#define FA_FWD_PP_AHEAD 4
#endif
// Block-sparse d = 64: one 128-key tile per 128-key block (no masked tiles there).
#ifndef FA_FWD_BC_SPARSE_D64
#define FA_FWD_BC_SPARSE_D64 128
#endif

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  const FwdKParams p = make_params(a);
  const dim3 grid((unsigned)(a.B * a.H * p.n_qblocks)), block(256);
  const bool sparse = a.block_mask != nullptr;
  const bool smask = a.causal || a.key_len != nullptr;
  timer_begin("fa_fwd_bf16", s);
  constexpr int BC128 = FA_FWD_BC_D128, BC64 = FA_FWD_BC_D64, BCS64 = FA_FWD_BC_SPARSE_D64;
  if (a.dropout.p8 && sparse) {
    // (the element masks are applied per tile as needed; with neither causal nor key_len no tile needs them)
    if (a.d == 128) fwd_bf16_kernel<128, BC128, true, true, true><<<grid, block, 0, s>>>(p);
    else fwd_bf16_kernel<64, BCS64, true, true, true><<<grid, block, 0, s>>>(p);
  } else if (a.dropout.p8) {
    if (a.d == 128) fwd_bf16_kernel<128, BC128, false, false, true><<<grid, block, 0, s>>>(p);
    else fwd_bf16_kernel<64, BC64, false, false, true><<<grid, block, 0, s>>>(p);
  } else if (a.d == 128) {
    if (sparse && smask) fwd_bf16_kernel<128, BC128, true, true><<<grid, block, 0, s>>>(p);
    else if (sparse) fwd_bf16_kernel<128, BC128, true><<<grid, block, 0, s>>>(p);
    else if (FA_FWD_PINGPONG) {
      FwdKParams pp = p;
      pp.n_qblocks = (a.N + kFwdRowsPP - 1) / kFwdRowsPP;
      fwd_pp_kernel<128, FA_FWD_PP_BC><<<dim3((unsigned)(a.B * a.H * pp.n_qblocks)), dim3(512), 0, s>>>(pp);
    } else fwd_bf16_kernel<128, BC128, false><<<grid, block, 0, s>>>(p);
  } else {
    if (sparse && smask) fwd_bf16_kernel<64, BCS64, true, true><<<grid, block, 0, s>>>(p);
    else if (sparse) fwd_bf16_kernel<64, BCS64, true><<<grid, block, 0, s>>>(p);
    else fwd_bf16_kernel<64, BC64, false><<<grid, block, 0, s>>>(p);
  }
  timer_end(s);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  const FwdKParams p = make_params(a);
  const dim3 grid((unsigned)(a.B * a.H * p.n_qblocks)), block(256);
  timer_begin("fa_fwd_f32", s);
  if (a.d == 128) fwd_f32_kernel<128><<<grid, block, 0, s>>>(p);
  else fwd_f32_kernel<64><<<grid, block, 0, s>>>(p);
  timer_end(s);
  return hipGetLastError();
}

}  // namespace fa
