// MFMA helpers for gfx950 (CDNA4): v_mfma_f32_32x32x16_bf16 operand types,
// packing, and the lane layout the attention kernels rely on.
//
// For C[32x32] += A[32x16] * B[16x32] with 64 lanes, lane l (h = l / 32):
//   A operand: row l % 32, k = 8h .. 8h+7   (8 bf16)
//   B operand: col l % 32, k = 8h .. 8h+7   (8 bf16)
//   C (16 f32): acc[4*I + J] = C[8*I + 4*h + J][l % 32], I, J in 0..3
// Because k is a summation index, A and B may present their k slots in any
// order as long as both use the same one; the kernels exploit this to feed
// an accumulator tile straight back in as the next product's operand.
#pragma once

#include "lh_internal.h"

namespace lh {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16 raw bytes
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// the same values as a two-term split: hi = bf16(x), lo = bf16(x - hi); the
// pair carries about 16 significant bits, so a product taken as
// hi*B + lo*B loses far less than one rounding of x to bf16
__device__ __forceinline__ void pack_split(const f32x16 &acc, int o, bf16x8 &hi, bf16x8 &lo) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f2 x = {acc[o + e], acc[o + e + 1]};
    const b2 h = __builtin_convertvector(x, b2);   // one packed convert per pair
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const f2 hf = {__uint_as_float(hb << 16), __uint_as_float(hb & 0xffff0000u)};
    const b2 l = __builtin_convertvector(x - hf, b2);
    hi[e] = h[0];
    hi[e + 1] = h[1];
    lo[e] = l[0];
    lo[e + 1] = l[1];
  }
}

// ---------------------------------------------------------------- row tiles
// A row tile X[r][n] (16-bit, D columns) in LDS is read two ways: as the
// "row" operand (lane % 32 = row r, k = columns 16s + 8h .. +7) and as the
// "column" operand (lane % 32 = column n, k = rows) with ds_read_b64_tr_b16.
// The transposing read hands lane 4a+b of each 16-lane group element b of
// the 8-byte pieces addressed by lanes a, a+4, a+8, a+12 of that group, so a
// group whose lane j points at row kbase + j/4, columns n0 + 4(j%4) receives
// column n0 + i of rows kbase..kbase+3 in its lane i.  16-byte chunks are
// XOR-swizzled per row (swz_r) so that both reads stay free of bank
// conflicts.
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Chunk permutation of row r.  LDS serves a 16-byte-per-lane read in
// passes of 16 lanes and the 8-byte transposing read in passes of 32 lanes
// (64 banks of 4 bytes).  A row-operand pass reads one chunk of each of 16
// consecutive rows; a transposing pass reads four consecutive chunks of each
// of 4 consecutive rows.  D = 128 (a row spans all banks): the low two row
// bits pick the 4-chunk group, bits 2-3 the chunk inside it, so both passes
// touch 16 distinct chunks.  D = 64 (two rows per bank line): row bit 1
// picks the group and bits 1-3 of the row, reversed, make rows of one parity
// distinct.
template <int D>
__device__ __forceinline__ int swz_r(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}
// element offset of (row r, column n) in a swizzled row tile
template <int D>
__device__ __forceinline__ int toff(int r, int n) {
  return r * D + ((((n >> 3) ^ swz_r<D>(r))) << 3) + (n & 7);
}
// row operand: row r, k-step s (columns 16s + 8h .. +7)
template <int D>
__device__ __forceinline__ bf16x8 ld_rowop(const bf16_t *X, int r, int s, int h) {
  return ld_bf16x8(X + toff<D>(r, 16 * s + 8 * h));
}
// column operand over the 32 columns nb .. nb+31, k-step s over rows, with
// k-slot 8h + 4u + J <-> row 16s + 8u + 4h + J (the order pack_split uses for
// an accumulator tile whose rows are 8I + 4h + J)
template <int D>
__device__ __forceinline__ bf16x8 ld_colop(const bf16_t *X, int s, int nb, int lane) {
  const int j = lane & 15, g = lane >> 4, h = lane >> 5;
  const int n = nb + 16 * (g & 1) + 4 * (j & 3);
  const int r = 16 * s + 4 * h + (j >> 2);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(X + toff<D>(r, n)));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(X + toff<D>(r + 8, n)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS traffic: waits for this wavefront's LDS
// operations only.  Outstanding global->LDS loads are not waited for here
// (a full __syncthreads fence would drain them all); callers wait for the
// loads they need with an explicit vmcnt first.  LDS data read after the
// barrier should be read through native vector types (f32x4, bf16x8): a
// read the backend splits and re-merges loses the memory information that
// tells it the read cannot overlap a pending global->LDS load, and it then
// waits for every such load.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// An accumulator tile "used" at this point: the MFMAs that form it cannot
// be moved below here by code motion (a scheduling fence alone does not stop
// it).  Emits nothing.
__device__ __forceinline__ void pin(const f32x16 &x) { asm volatile("" ::"a"(x)); }
// the same, for a tile that stays in VGPRs
__device__ __forceinline__ void pin_v(const f32x16 &x) { asm volatile("" ::"v"(x)); }

// Issue-order prescription for the scheduler, within one fenced region: NM
// MFMAs, the first RG of them each followed by NR LDS reads (reads started
// early, under MFMAs that do not need them), every one followed by NV VALU
// instructions (transcendentals included; NV = 0: VALU left unconstrained).
// Groups the region cannot fill are skipped.
template <int NM, int RG, int NR, int NV>
__device__ __forceinline__ void sched_mix() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < RG) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
  }
}

// Raw buffer resource over `nbytes` bytes at `p` (word 3: 32-bit data
// format, as gfx9 raw buffer accesses require).  Global->LDS copies go
// through buffer loads rather than global (FLAT) loads: an outstanding FLAT
// load that writes LDS makes the compiler treat the LDS counter as out of
// order and wait for every LDS read at the first use of any of them, while
// buffer loads leave LDS reads counted in order.  Loads past `nbytes` read
// zeros.
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc make_rsrc(const void *p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)nbytes,
                                           0x00020000);
}
// one head's subsequence rows (S x d) and its transposed copy (d x Sp) in
// bf16 fit a buffer resource's 31-bit byte range
inline bool rsrc_fits(const Geo &g) {
  return (int64_t)g.S * g.d * 2 <= INT32_MAX && (int64_t)g.Sp * g.d * 2 <= INT32_MAX;
}
// async copy of `bytes` (4 or 16) at byte offset `off` of `r` into LDS at
// `dst` + 4 or 16 x lane (dst uniform over the wavefront)
template <int BYTES>
__device__ __forceinline__ void lds_dma(brsrc r, void *dst, uint32_t off) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte pieces");
  if constexpr (BYTES == 16) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, off, 0, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 4, off, 0, 0, 0);
  }
}

// Async global -> LDS copies of ROWS-row blocks of a [*, D] bf16 matrix
// (row stride D, read through a buffer resource) into swizzled row tiles,
// by the NTHR threads t = 0..NTHR-1 (whole wavefronts, each issuing the same
// number of 1 KB pieces).  The per-thread source offsets within a block are
// fixed, so they are computed once; a block then costs one add per piece.
// Rows past the resource's end read as zeros.
template <int D, int ROWS, int NTHR>
struct TileMap {
  static constexpr int WAVES = NTHR / 64;
  static constexpr int PIECES = ROWS * D / 8 / 64;
  static_assert(PIECES % WAVES == 0, "pieces split evenly over the wavefronts");
  static constexpr int NP = PIECES / WAVES;
  uint32_t off[NP];   // byte offset of this thread's 16 bytes of piece i
  int w;              // wavefront index (uniform)
  __device__ __forceinline__ void init(int t) {
    const int lane = t & 63;
    w = __builtin_amdgcn_readfirstlane(t >> 6);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int chunk = (w + i * WAVES) * 64 + lane;
      const int r = chunk / (D / 8), p = chunk % (D / 8);
      off[i] = (uint32_t)((r * D + (p ^ swz_r<D>(r)) * 8) * 2);
    }
  }
  // rows row0 .. row0 + ROWS - 1 of `src` into the tile at `dst`
  __device__ __forceinline__ void load(bf16_t *dst, brsrc src, int64_t row0) const {
    const uint32_t base = (uint32_t)(row0 * D * 2);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      lds_dma<16>(src, reinterpret_cast<unsigned char *>(dst) + (w + i * WAVES) * 1024,
                  base + off[i]);
  }
};

// ---------------------------------------------------------------- key rings
// The dQ and forward kernels stream key blocks of 32 rows (K, V and each
// key's mask bias) through an LDS ring; the REDUNDANT flags of a
// workgroup's key range are kept as bits.
constexpr int kKeyBlock = 32;
constexpr size_t kMaxLds = 160 * 1024;   // LDS of one CU

template <int D>
struct KeyStage {
  bf16_t k[kKeyBlock * D];   // K rows of the block
  bf16_t v[kKeyBlock * D];   // V rows
  float bias[kKeyBlock];     // 0, or -inf for a redundant key or one past the range
};

// REDUNDANT bits of keys 0 .. kend-1 of one (b, h) into `bits` (one 64-bit
// word per 64 keys): each wavefront of the NTHR threads packs 64-key chunks
// with a ballot, 16 flag loads in flight per lane.  Readers need a barrier.
template <int NTHR>
__device__ __forceinline__ void stage_flag_bits(uint64_t *bits, const uint8_t *flags,
                                                int64_t kend, int w, int lane) {
  constexpr int FPT = 16, WAVES = NTHR / 64;
  const int64_t nch = (kend + 63) / 64;
  for (int64_t c0 = 0; c0 < nch; c0 += (int64_t)FPT * WAVES) {
    uint8_t v[FPT];
#pragma unroll
    for (int j = 0; j < FPT; ++j) {
      const int64_t i = (c0 + (int64_t)j * WAVES + w) * 64 + lane;
      v[j] = i < kend ? flags[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < FPT; ++j) {
      const int64_t c = c0 + (int64_t)j * WAVES + w;   // uniform over the wavefront
      const uint64_t m = __ballot((v[j] & LH_ROW_REDUNDANT) != 0);
      if (c < nch && lane == 0) bits[c] = m;
    }
  }
}

// the bias of key kk from the staged bits (keys at or past kend are masked)
__device__ __forceinline__ float key_bias(const uint64_t *bits, int64_t kk, int64_t kend) {
  const bool red = kk >= kend || ((bits[kk >> 6] >> (kk & 63)) & 1u);
  return red ? -INFINITY : 0.f;
}

// the values of lanes l and l ^ 32 exchanged (v_permlane32_swap)
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32);
}

}  // namespace lh
