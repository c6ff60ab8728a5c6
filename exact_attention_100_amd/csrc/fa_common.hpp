// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the CDNA4 bf16 / fp32 matrix-core (MFMA) operations, fast
// exp2 / log2, bf16 packing and the workgroup -> tile schedule.
//
// MFMA register layouts used throughout (64-lane wavefront, 32x32 output):
//   A operand (32 x K):  lane l holds row (l % 32); its K values are the slots
//                        of lane group g = l / 32.
//   B operand (K x 32):  lane l holds column (l % 32), slots of group g.
//   C / D (32 x 32 f32): lane l holds column (l % 32); register r holds row
//                        8 * (r / 4) + 4 * g + (r % 4).
// Which K index a (group, slot) pair stands for is our choice, as long as the
// A and B operands of one instruction make the same choice; every kernel
// documents the choice it makes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16)
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, f32) += A(32x2, f32) * B(2x32, f32); lane group g holds K index g.
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round two floats to bf16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight floats -> bf16x8 operand (element i = f[i]).
__device__ __forceinline__ bf16x8 pack_bf16x8(float f0, float f1, float f2, float f3, float f4,
                                              float f5, float f6, float f7) {
  u32x4 u;
  u[0] = pack_bf16x2(f0, f1);
  u[1] = pack_bf16x2(f2, f3);
  u[2] = pack_bf16x2(f4, f5);
  u[3] = pack_bf16x2(f6, f7);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 concat_bf16x4(bf16x4 lo, bf16x4 hi) {
  u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 u;
  u[0] = a[0];
  u[1] = a[1];
  u[2] = b[0];
  u[3] = b[1];
  return __builtin_bit_cast(bf16x8, u);
}

// Combine a value with the one held by lane (l ^ 32), the lane holding the same
// MFMA column in the other lane group, through v_permlane32_swap (lanes < 32 get
// {own, partner}, lanes >= 32 get {partner, own}; max and sum are symmetric).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Build the low/high bf16 halves of four packed bf16 pairs into two 4-element
// rows: in[j] = (x_j, y_j) -> xs = (x_0..x_3), ys = (y_0..y_3).
__device__ __forceinline__ void split_pairs4(uint32_t in0, uint32_t in1, uint32_t in2, uint32_t in3,
                                             u32x2& xs, u32x2& ys) {
  xs[0] = (in0 & 0xFFFFu) | (in1 << 16);
  xs[1] = (in2 & 0xFFFFu) | (in3 << 16);
  ys[0] = (in0 >> 16) | (in1 & 0xFFFF0000u);
  ys[1] = (in2 >> 16) | (in3 & 0xFFFF0000u);
}

// Transposing LDS read (ds_read_b64_tr_b16). For a row-major bf16 matrix X[k][m]
// in LDS with row stride ld (elements), lane l receives the 8 values
//   X[k0 + kmap(g, s)][m0 + l % 32],  s = 0..7,  g = l / 32,
//   kmap(g, s) = 4 g + s (s < 4),  8 + 4 g + (s - 4) (s >= 4),
// i.e. a 32 x 16 operand (rows m, K index k) whose slot order matches the rows of
// an MFMA accumulator (register r <-> row 8 (r/4) + 4 g + r % 4). The hardware
// gives lane j of each 16-lane group element (j % 4) of the 8-byte chunks
// addressed by lanes 4 t + j / 4 (t = 0..3), so the 16 lanes of a group address
// a 4-row x 16-column block and each receives one of its columns.
__device__ __forceinline__ bf16x8 lds_read_tr_k16(const bf16* X, int ld, int k0, int m0, int lane) {
  const int g = lane >> 5, h = (lane >> 4) & 1, j = lane & 15;
  const bf16* p0 = X + (k0 + 4 * g + (j >> 2)) * ld + m0 + 16 * h + 4 * (j & 3);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 8 * ld));
  return concat_bf16x4(lo, hi);
}

// Swizzled row-major LDS tiles. A tile with COLS bf16 columns (COLS / 8 chunks
// of 16 bytes per row, no padding) stores element (r, c) in chunk
// (c / 8) ^ tile_swz<COLS>(r) of row r. tile_swz is linear over GF(2) in the low
// four row bits; the maps below keep three access patterns free of bank
// conflicts (checked for both 32- and 64-bank LDS models): 16-byte row reads by
// 16 consecutive rows (MFMA operands), transposing 8-byte reads of 4 rows x 32
// columns (lds_read_tr_k16_swz) and 16-byte row-major writes.
template <int COLS>
__device__ __forceinline__ int tile_swz(int r) {
  static_assert(COLS == 128 || COLS == 64 || COLS == 32, "unsupported tile width");
  constexpr int b0 = COLS == 128 ? 4 : (COLS == 64 ? 2 : 0);
  constexpr int b1 = COLS == 128 ? 10 : (COLS == 64 ? 4 : 2);
  return ((r & 1) ? b0 : 0) ^ ((r & 2) ? b1 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
}
template <int COLS>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * COLS + ((((c >> 3) ^ tile_swz<COLS>(r))) << 3) + (c & 7);
}

// lds_read_tr_k16 on a swizzled tile (same result layout).
template <int COLS>
__device__ __forceinline__ bf16x8 lds_read_tr_k16_swz(const bf16* X, int k0, int m0, int lane) {
  const int g = lane >> 5, h = (lane >> 4) & 1, j = lane & 15;
  const int r = k0 + 4 * g + (j >> 2), c = m0 + 16 * h + 4 * (j & 3);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(X + tile_off<COLS>(r, c)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(X + tile_off<COLS>(r + 8, c)));
  return concat_bf16x4(lo, hi);
}

// Direct global -> LDS copies of a [ROWS x COLS] bf16 tile into the swizzled
// layout above (global_load_lds_dwordx4: lane i of an instruction writes LDS
// chunk base + i, so each lane fetches the global chunk that belongs there).
// The per-lane source offsets are computed once (init); issue() then costs one
// address add per copy for a full tile. Rows row0 + r at or past nvalid are
// clamped to row nvalid - 1 (the callers only ever give such rows probability
// 0 or discard what they produce). NWAVES waves share a copy; the caller waits
// (vmcnt) and synchronises before the tile is read.
template <int ROWS, int COLS, int NWAVES>
struct TileCopy {
  static constexpr int CPR = COLS / 8;
  static constexpr int PER_WAVE = ROWS * CPR / (64 * NWAVES);
  static_assert(PER_WAVE >= 1 && PER_WAVE * 64 * NWAVES == ROWS * CPR, "tile must split into whole wave copies");
  // Lane offsets are unsigned 32-bit byte offsets: the API admits row strides below 2^23
  // elements, so 256 rows at most (255 (2^23 - 16) 2 + 256 bytes < 2^32).
  static_assert(ROWS <= 256, "32-bit lane offsets cover 256 rows of the largest admitted stride");
  uint32_t offb[PER_WAVE];  // byte offset of this lane's source chunk from the tile's first row
  int32_t row[PER_WAVE];    // tile row of that chunk
  int wave;               // wave index (uniform)

  __device__ __forceinline__ void init(int wave_uniform, int lane, int64_t ld) {
    wave = wave_uniform;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int pch = (i * NWAVES + wave) * 64 + lane;
      row[i] = pch / CPR;
      offb[i] = (uint32_t)(2 * (row[i] * ld + 8 * ((pch % CPR) ^ tile_swz<COLS>(row[i]))));
    }
  }
  __device__ __forceinline__ void issue(bf16* lds_tile, const bf16* g, int64_t ld, int row0, int nvalid) const {
    typedef const void __attribute__((address_space(1)))* gptr;
    typedef void __attribute__((address_space(3)))* lptr;
    const bf16* gt = g + (int64_t)row0 * ld;
    // (opaque per issue: each copy's LDS destination, the M0 operand, is re-formed from
    // it by a scalar add instead of being kept in a scalar register across the loop)
    int wv = wave;
    asm volatile("" : "+s"(wv));
    // Each copy addresses a scalar base plus this lane's unsigned 32-bit byte offset (the
    // saddr form: no vector address arithmetic per copy of a full tile).
    const char* gb = reinterpret_cast<const char*>(gt);
    if (row0 + ROWS <= nvalid) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i)
        __builtin_amdgcn_global_load_lds((gptr)(gb + offb[i]), (lptr)(lds_tile + 8 * 64 * (i * NWAVES + wv)), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        // Step back over rows past nvalid - 1 (at most row[i] of them, so the offset
        // stays non-negative and within 32 bits).
        const int over = max(row0 + row[i] - (nvalid - 1), 0);
        __builtin_amdgcn_global_load_lds((gptr)(gb + (offb[i] - (uint32_t)(2 * over * ld))),
                                         (lptr)(lds_tile + 8 * 64 * (i * NWAVES + wv)), 16, 0, 0);
      }
    }
  }
};

// LDS reads issued as inline assembly, for loops that manage their own waits.
// While a direct global -> LDS copy is in flight the compiler only ever waits
// for all LDS reads at once (lgkmcnt(0)); LDS reads return in order and those
// copies are counted by vmcnt alone, so a loop that knows how many reads it
// issued after the one it needs can wait for exactly that one (lds_wait). The
// byte offset `off` must fold to a constant; the common tile offsets become the
// instruction's immediate. The caller makes sure (barriers) the data is there.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// Every multiple of 1 KiB the 16-bit offset field holds (buffer + block offsets of the tile reads).
#define FA_DS_OFFSETS(X) \
  X(0) X(1024) X(2048) X(3072) X(4096) X(5120) X(6144) X(7168) \
  X(8192) X(9216) X(10240) X(11264) X(12288) X(13312) X(14336) X(15360) \
  X(16384) X(17408) X(18432) X(19456) X(20480) X(21504) X(22528) X(23552) \
  X(24576) X(25600) X(26624) X(27648) X(28672) X(29696) X(30720) X(31744) \
  X(32768) X(33792) X(34816) X(35840) X(36864) X(37888) X(38912) X(39936) \
  X(40960) X(41984) X(43008) X(44032) X(45056) X(46080) X(47104) X(48128) \
  X(49152) X(50176) X(51200) X(52224) X(53248) X(54272) X(55296) X(56320) \
  X(57344) X(58368) X(59392) X(60416) X(61440) X(62464) X(63488) X(64512)
__device__ __forceinline__ bf16x8 lds_read_b128_asm(uint32_t addr, int off) {
  u32x4 v;
  switch (off) {
#define FA_CASE(O) \
  case O:          \
    asm volatile("ds_read_b128 %0, %1 offset:" #O : "=v"(v) : "v"(addr)); \
    break;
    FA_DS_OFFSETS(FA_CASE)
#undef FA_CASE
    default:
      asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr + off));
  }
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x4 lds_read_tr_asm(uint32_t addr, int off) {
  u32x2 v;
  switch (off) {
#define FA_CASE(O) \
  case O:          \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:" #O : "=v"(v) : "v"(addr)); \
    break;
    FA_DS_OFFSETS(FA_CASE)
#undef FA_CASE
    default:
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr + off));
  }
  return __builtin_bit_cast(bf16x4, v);
}
// s_waitcnt lgkmcnt(n) (vmcnt and expcnt left alone); n must fold to a constant.
// Calls f(std::integral_constant<int, i>) for i = 0 .. N - 1 in order: a loop whose
// index is a compile-time constant in the body, whatever the body's size.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Four consecutive floats of a per-row statistics vector (LDS), as inline assembly
// like the tile reads; off is one of the row-group offsets below.
#define FA_DS_STAT_OFFSETS(X) X(0) X(32) X(64) X(96) X(128) X(160) X(192) X(224)
__device__ __forceinline__ f32x4 lds_read_f32x4_asm(uint32_t addr, int off) {
  f32x4 v;
  switch (off) {
#define FA_CASE(O) \
  case O:          \
    asm volatile("ds_read_b128 %0, %1 offset:" #O : "=v"(v) : "v"(addr)); \
    break;
    FA_DS_STAT_OFFSETS(FA_CASE)
#undef FA_CASE
    default:
      asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr + off));
  }
  return v;
}
__device__ __forceinline__ void lds_wait(int n) {
  switch (n) {
#define FA_W(N) \
  case N:       \
    __builtin_amdgcn_s_waitcnt(0xC07F | ((N) << 8)); \
    break;
    FA_W(0) FA_W(1) FA_W(2) FA_W(3) FA_W(4) FA_W(5) FA_W(6) FA_W(7)
    FA_W(8) FA_W(9) FA_W(10) FA_W(11) FA_W(12) FA_W(13) FA_W(14)
#undef FA_W
    default:
      __builtin_amdgcn_s_waitcnt(0xC07F | (15 << 8));
  }
}

// Loop-invariant per-lane byte offsets into swizzled [rows x COLS] bf16 tiles
// (bytes, so that an LDS address is the offset plus an immediate).
// Row reads: the MFMA A operand of rows 32 b + l32 at k-step kk (16 columns,
// lane group g taking columns 8 g .. 8 g + 7) lives at element
// b * 32 * COLS + row[kk] / 2 (the swizzle depends only on the row's low four bits).
// Transposing reads (lds_read_tr_k16_swz) at k0 = 16 ks, m0 = 32 mb read
// elements 16 ks * COLS + tr_lo[mb] / 2 and 16 ks * COLS + tr_hi[mb] / 2.
template <int COLS>
struct TileOffsets {
  int32_t row[COLS / 16];
  int32_t tr_lo[COLS / 32], tr_hi[COLS / 32];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5, h = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int kk = 0; kk < COLS / 16; ++kk) row[kk] = 2 * tile_off<COLS>(l32, 16 * kk + 8 * g);
    const int r = 4 * g + (j >> 2);
#pragma unroll
    for (int mb = 0; mb < COLS / 32; ++mb) {
      const int c = 32 * mb + 16 * h + 4 * (j & 3);
      tr_lo[mb] = 2 * tile_off<COLS>(r, c);
      tr_hi[mb] = 2 * tile_off<COLS>(r + 8, c);
    }
  }
  // Makes the offsets opaque to the optimiser at this point. Called once per
  // loop iteration, it keeps buffer + offset sums from being hoisted out of the
  // loop as separate registers per buffer: each read then adds the buffer's
  // static base as the LDS instruction's immediate offset instead.
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < COLS / 16; ++i) asm volatile("" : "+v"(row[i]));
#pragma unroll
    for (int i = 0; i < COLS / 32; ++i) asm volatile("" : "+v"(tr_lo[i]), "+v"(tr_hi[i]));
  }
  __device__ __forceinline__ bf16x8 read_row(const bf16* X, int b, int kk) const {
    const char* p = reinterpret_cast<const char*>(X + b * 32 * COLS) + row[kk];
    return *reinterpret_cast<const bf16x8*>(p);
  }
  // The same reads as inline assembly (lds_read_*_asm; base = lds_address of X):
  // the caller waits for them itself (lds_wait).
  __device__ __forceinline__ bf16x8 read_row_asm(uint32_t base, int b, int kk) const {
    return lds_read_b128_asm(base + row[kk], b * 64 * COLS);
  }
  __device__ __forceinline__ bf16x8 read_tr_asm(uint32_t base, int ks, int mb) const {
    return concat_bf16x4(lds_read_tr_asm(base + tr_lo[mb], 32 * ks * COLS),
                         lds_read_tr_asm(base + tr_hi[mb], 32 * ks * COLS));
  }
  __device__ __forceinline__ bf16x8 read_tr(const bf16* X, int ks, int mb) const {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const char* p = reinterpret_cast<const char*>(X + 16 * ks * COLS);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + tr_lo[mb]));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + tr_hi[mb]));
    return concat_bf16x4(lo, hi);
  }
};

// The same per-lane offsets with one LDS array's address already added (computed once):
// reads of the tile buffers inside that array then name the buffer through the
// instruction's immediate offset only, so no address arithmetic is repeated per tile.
template <int COLS>
struct TileAddr {
  uint32_t row[COLS / 16];
  uint32_t tr_lo[COLS / 32], tr_hi[COLS / 32];
  __device__ __forceinline__ void init(const TileOffsets<COLS>& to, uint32_t array_base) {
#pragma unroll
    for (int i = 0; i < COLS / 16; ++i) row[i] = array_base + (uint32_t)to.row[i];
#pragma unroll
    for (int i = 0; i < COLS / 32; ++i) {
      tr_lo[i] = array_base + (uint32_t)to.tr_lo[i];
      tr_hi[i] = array_base + (uint32_t)to.tr_hi[i];
    }
  }
  // buf: byte offset of the tile buffer in the array (folds to a constant).
  __device__ __forceinline__ bf16x8 read_row(int buf, int b, int kk) const {
    return lds_read_b128_asm(row[kk], buf + b * 64 * COLS);
  }
  __device__ __forceinline__ bf16x8 read_tr(int buf, int ks, int mb) const {
    return concat_bf16x4(lds_read_tr_asm(tr_lo[mb], buf + 32 * ks * COLS),
                         lds_read_tr_asm(tr_hi[mb], buf + 32 * ks * COLS));
  }
  // The same read from a buffer chosen at run time: its offset goes into the
  // address (one add per read) and the immediate keeps only the constant part,
  // where read_tr would branch over the possible immediates.
  __device__ __forceinline__ bf16x8 read_tr_rt(uint32_t buf, int ks, int mb) const {
    return concat_bf16x4(lds_read_tr_asm(tr_lo[mb] + buf, 32 * ks * COLS),
                         lds_read_tr_asm(tr_hi[mb] + buf, 32 * ks * COLS));
  }
};

// Two-sided element mask with one compare per entry: offsets off (compile-time
// constants) are kept iff lo <= off <= hi. As unsigned numbers, off - lo <= hi - lo
// exactly when lo <= off <= hi (for hi >= lo); an empty range becomes one that no
// offset reaches. Each entry's compare then goes straight to VCC instead of two
// lane masks per entry held in scalar registers.
struct RangeMask {
  uint32_t lo, span;
  __device__ __forceinline__ RangeMask(int lo_, int hi_) {
    const bool empty = hi_ < lo_;
    lo = empty ? 0x40000000u : (uint32_t)lo_;
    span = empty ? 0u : (uint32_t)(hi_ - lo_);
  }
  __device__ __forceinline__ bool keep(int off) const { return (uint32_t)off - lo <= span; }
};

// A wave's 32 x D bf16 output rows through LDS, so that the global stores are whole rows.
// In the MFMA accumulator layout lane l holds row l % 32 and, for block db and register
// quad j, the 4 values at columns 32 db + 8 j + 4 (l / 32) (packed in w[db][j]): stored
// straight to memory, every store instruction writes 8 bytes into each of 32 rows. Here
// each lane writes its pieces into a wave-private LDS slice (16-byte chunks swizzled by
// row, so neither the 8-byte writes nor the 16-byte reads meet bank conflicts), then
// reads back whole 16-byte chunks in row order: each global store covers complete rows
// (64 lanes x 16 bytes, D / 8 lanes per row). Rows at or past nvalid are not stored.
// slice: 32 * D * 2 bytes of LDS no other wave touches meanwhile.
template <int D>
__device__ __forceinline__ void store_rows_via_lds(bf16* slice, const u32x2 (&w)[D / 32][4], bf16* out, int64_t ld,
                                                   int row0, int nvalid, int lane) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  // (opaque: the addresses below are formed here, after the caller's loops, instead of
  // being hoisted into registers held across them)
  asm volatile("" : "+v"(lane));
  const int r = lane & 31, h = lane >> 5;
  char* sl = reinterpret_cast<char*>(slice);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * db + j;
      *reinterpret_cast<u32x2*>(sl + r * (2 * D) + 16 * (c ^ (r % CPR)) + 8 * h) = w[db][j];
    }
  // (the reads below take other lanes' writes: keep them after the writes)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // Instruction i reads chunk cc of row rr0 + RPI i (RPI = 64 / CPR rows per instruction).
  constexpr int RPI = 64 / CPR;
  const int rr0 = lane / CPR, cc = lane % CPR;
  u32x4 v[CPR / 2];
#pragma unroll
  for (int i = 0; i < CPR / 2; ++i) {
    const int rr = rr0 + RPI * i;
    v[i] = *reinterpret_cast<const u32x4*>(sl + rr * (2 * D) + 16 * (cc ^ (rr % CPR)));
  }
  bf16* o = out + (int64_t)(row0 + rr0) * ld + 8 * cc;
#pragma unroll
  for (int i = 0; i < CPR / 2; ++i)
    if (row0 + rr0 + RPI * i < nvalid) *reinterpret_cast<u32x4*>(o + (int64_t)(RPI * i) * ld) = v[i];
}

// Dropout keep bits from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011): 4 x 32-bit counter, 2 x 32-bit
// key, ten rounds of two 32 x 32 -> 64-bit products mixed by XOR, the key bumped
// by the Weyl constants between rounds. The pair (query i, key j) of instance
// bh takes byte (j mod 4) of word (i mod 4) at counter (i div 4, j div 4, bh,
// offset) and is kept iff that byte is >= p8 (drop probability p8 / 256), so
// one call serves a 4 x 4 block of pairs.
struct Dropout {
  uint32_t p8;       // 1..255 (0: the kernels are built without dropout)
  uint32_t k0, k1;   // seed, low and high words
  uint32_t offset;   // counter word 3
  float scale;       // 1 / (1 - p8 / 256)
};
// The generator as a state that advances one round at a time, so that its work can be
// spread over other instructions.
struct Philox {
  uint32_t c0, c1, c2, c3, k0, k1;
  __device__ __forceinline__ void round(int r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
};
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
  Philox g{c0, c1, c2, c3, k0, k1};
#pragma unroll
  for (int r = 0; r < 10; ++r) g.round(r);
  u32x4 r;
  r[0] = g.c0;
  r[1] = g.c1;
  r[2] = g.c2;
  r[3] = g.c3;
  return r;
}
// Lane r of each group of four lanes receives v from lane r ^ k (k = 1, 2, 3; DPP).
__device__ __forceinline__ uint32_t quad_xor(uint32_t v, int k) {
  return k == 1 ? (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false)    // [1,0,3,2]
                : (k == 2 ? (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false)   // [2,3,0,1]
                          : (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xF, 0xF, false));  // [3,2,1,0]
}

// The generator state of this lane's call for key quads c0 .. c0 + 3 (see below).
__device__ __forceinline__ Philox dropout_row_state(const Dropout& d, int i, int key0, uint32_t bh, int c0) {
  const int t = i & 3;
  return Philox{(uint32_t)i >> 2, (uint32_t)(key0 + 8 * (c0 + t)) >> 2, bh, d.offset, d.k0, d.k1};
}
// Words c0 .. c0 + 3 of the keep words below from that call's output.
template <int NC>
__device__ __forceinline__ void dropout_row_words_of(int i, const Philox& w, int c0, uint32_t (&out)[NC]) {
  const int t = i & 3;
  const uint32_t wr[4] = {w.c0, w.c1, w.c2, w.c3};
  uint32_t got[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int want = t ^ k;  // the word the partner lane (t ^ k) needs
    const uint32_t send = want == 0 ? wr[0] : (want == 1 ? wr[1] : (want == 2 ? wr[2] : wr[3]));
    got[k] = k == 0 ? send : quad_xor(send, k);  // my word of quad c0 + (t ^ k)
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = j ^ t;
    out[c0 + j] = k == 0 ? got[0] : (k == 1 ? got[1] : (k == 2 ? got[2] : got[3]));
  }
}
// Keep words of NC key quads (keys key0 + 8 c .. + 3) for this lane's query i,
// where the four lanes of each lane quad hold queries 4 m .. 4 m + 3 (i mod 4 =
// lane mod 4). The four lanes need the same generator calls (one word each), so
// each lane computes one call in four and the words are exchanged within the
// quad. All 64 lanes must be active.
template <int NC>
__device__ __forceinline__ void dropout_row_words(const Dropout& d, int i, int key0, uint32_t bh,
                                                  uint32_t (&out)[NC]) {
  static_assert(NC % 4 == 0, "key quads come in groups of four");
#pragma unroll
  for (int c0 = 0; c0 < NC; c0 += 4) {
    Philox g = dropout_row_state(d, i, key0, bh, c0);
#pragma unroll
    for (int r = 0; r < 10; ++r) g.round(r);
    dropout_row_words_of<NC>(i, g, c0, out);
  }
}

// Keep bits of this lane's key j for NC query quads (queries q4 + 8 c .. + 3):
// bit 4 c + w is query q4 + 8 c + w. The four lanes of each lane quad hold keys
// 4 m .. 4 m + 3 (j mod 4 = lane mod 4) and need the same calls (one byte of
// each word), so each lane computes one call in four, reduces it to its 4 x 4
// keep bits and hands each partner its column. All 64 lanes must be active.
// The generator state of this lane's call for query quads c0 .. c0 + 3 (see below).
__device__ __forceinline__ Philox dropout_col_state(const Dropout& d, int j, int q4, uint32_t bh, int c0) {
  const int t = j & 3;
  return Philox{(uint32_t)(q4 + 8 * (c0 + t)) >> 2, (uint32_t)j >> 2, bh, d.offset, d.k0, d.k1};
}
// Bits 4 c0 .. 4 c0 + 15 of the keep bits below from that call's output words.
__device__ __forceinline__ uint32_t dropout_col_bits_of(const Dropout& d, int j, const Philox& w, int c0) {
  const int t = j & 3;
  const uint32_t wr[4] = {w.c0, w.c1, w.c2, w.c3};
  uint32_t kb = 0;  // bit 4 b + r: key byte b of query row r kept
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int b = 0; b < 4; ++b) kb |= (((wr[r] >> (8 * b)) & 0xFFu) >= d.p8 ? 1u : 0u) << (4 * b + r);
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t send = (kb >> (4 * (t ^ k))) & 0xFu;  // the partner's key column
    const uint32_t got = k == 0 ? send : quad_xor(send, k);
    bits |= got << (4 * (c0 + (t ^ k)));
  }
  return bits;
}
template <int NC>
__device__ __forceinline__ uint32_t dropout_col_bits(const Dropout& d, int j, int q4, uint32_t bh) {
  static_assert(NC % 4 == 0 && NC <= 8, "query quads come in groups of four, 32 bits at most");
  uint32_t bits = 0;
#pragma unroll
  for (int c0 = 0; c0 < NC; c0 += 4) {
    Philox g = dropout_col_state(d, j, q4, bh, c0);
#pragma unroll
    for (int r = 0; r < 10; ++r) g.round(r);
    bits |= dropout_col_bits_of(d, j, g, c0);
  }
  return bits;
}

// 0xFFFF in each 16-bit half of a packed bf16 pair whose pair is kept: bytes c
// and c + 1 of `w` against p8.
__device__ __forceinline__ uint32_t dropout_pair_mask(uint32_t w, int c, uint32_t p8) {
  const uint32_t lo = ((w >> (8 * c)) & 0xFFu) >= p8 ? 0x0000FFFFu : 0u;
  const uint32_t hi = ((w >> (8 * c + 8)) & 0xFFu) >= p8 ? 0xFFFF0000u : 0u;
  return lo | hi;
}
// Zeroes the dropped entries of an 8-value packed operand holding two key quads
// (words w_a for values 0..3, w_b for values 4..7).
__device__ __forceinline__ bf16x8 dropout_apply8(bf16x8 v, uint32_t w_a, uint32_t w_b, uint32_t p8) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u[0] &= dropout_pair_mask(w_a, 0, p8);
  u[1] &= dropout_pair_mask(w_a, 2, p8);
  u[2] &= dropout_pair_mask(w_b, 0, p8);
  u[3] &= dropout_pair_mask(w_b, 2, p8);
  return __builtin_bit_cast(bf16x8, u);
}

// Compile-time flag for generic lambdas (selects the masked / unmasked variant
// of a tile body without per-element branches).
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int uniform_wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Same for a vector of COUNT (<= 64) floats: one copy by one wave; lanes past
// COUNT write the padding of a 64-float LDS array.
__device__ __forceinline__ void vec_dma64(float* lds_vec, const float* g, int i0, int nvalid, int lane) {
  const int64_t gi = min(i0 + lane, nvalid - 1);
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(g + gi),
                                   (void __attribute__((address_space(3)))*)(lds_vec), 4, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (including
// direct-to-LDS copies) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Block-sparse attention: the kept blocks along one line of an nb x nb block
// mask, in increasing order, written to `list` (LDS). ROW: mask[line][j], the
// key blocks seen by query block `line`; otherwise mask[j][line], the query
// blocks that see key block `line`. With causal, blocks above the diagonal (key
// block > query block) are dropped: every entry of them is masked. Wave 0 loads
// the line (all of its loads issued before the first is used) and forms the list
// with ballots; after a workgroup barrier every thread gets the count. Every
// thread of the workgroup must call it. nb <= kMaxBlocks.
constexpr int kMaxBlocks = 1024;
template <bool ROW>
__device__ __forceinline__ int kept_block_list(const uint8_t* mask, int nb, int line, int causal, int16_t* list,
                                               int* count) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    constexpr int K = kMaxBlocks / 64;
    uint32_t m[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = 64 * k + lane;
      m[k] = 0;
      if (j < nb) m[k] = ROW ? mask[(int64_t)line * nb + j] : mask[(int64_t)j * nb + line];
    }
    int n = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (64 * k < nb) {  // uniform
        const int j = 64 * k + lane;
        const bool keep = j < nb && m[k] != 0 && (!causal || (ROW ? j <= line : j >= line));
        const uint64_t bal = __ballot(keep);
        if (keep) list[n + __popcll(bal & ((1ull << lane) - 1ull))] = (int16_t)j;
        n += __popcll(bal);
      }
    }
    if (lane == 0) *count = n;
  }
  __syncthreads();
  return *count;
}

// Workgroup -> (instance, tile) schedule. Consecutive workgroup ids are handed
// to the 8 XCDs in turn; when the instance count allows it, all tiles of one
// (batch, head) instance go to the same XCD so its K/V (or Q/dO) re-reads hit
// that XCD's L2. Tiles are issued in `rank` order; the caller turns the rank
// into a tile index (e.g. heaviest tile first).
__device__ __forceinline__ void schedule_tile(int bid, int n_inst, int n_tiles, int& inst, int& rank) {
  if ((n_inst & 7) == 0) {
    const int xcd = bid & 7, idx = bid >> 3, per = n_inst >> 3;
    rank = idx / per;
    inst = xcd * per + (idx - rank * per);
  } else {
    rank = bid / n_inst;
    inst = bid - rank * n_inst;
  }
  (void)n_tiles;
}

}  // namespace fa
