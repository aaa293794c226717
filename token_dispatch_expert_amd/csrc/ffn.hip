// Expert FFN forward and backward on gfx950: grouped GEMMs on MFMA with the
// row gather fused into the operand loads, the SiLU / SwiGLU activation in
// the epilogues, and a deterministic gate-weighted combine.
//
// What is computed follows the MoEBlaze wiki note, "Core method":
//   - "materialisation-free token dispatch": the expert MLP reads its input
//     rows straight from the original (L, d) tensor through
//     expert_token_indices; the second-MLP output is written back into
//     (L, d) through the token-side indices; backward scatters the (L, d)
//     gradient through the same indices and accumulates the input gradient
//     on the fly, with no (L*K, d) buffer in either direction;
//   - "SwiGLU kernel fusion + activation checkpoint": both first-layer
//     projections share one load of x, SiLU(a)*b is formed in registers,
//     only A and B are kept, and backward recomputes SiLU(A) from them; the
//     input gradients of both branches are summed inside one GEMM over the
//     concatenated [dA | dB] x [W1 | W3]^T.
//
// GEMM engine (all six GEMMs): a 256 x 256 output tile per 512-thread
// workgroup; eight wavefronts (two per SIMD) in a 2 x 4 grid, each owning
// 128 x 64 = 4 x 2 MFMA 32x32 tiles (bf16: v_mfma_f32_32x32x16_bf16;
// float32: four v_mfma_f32_32x32x2f32 per 8-element k group).  One k-tile is
// 128 bytes of k per row (64 bf16 / 32 float32).  Operands are copied from
// global memory straight into LDS (global_load_lds, 16 bytes per lane), the
// next k-tile's copies issued before the current tile's MFMAs; LDS is double
// buffered (128 KB).  MFMA fragments for k-chunk kc + 1 are read while the
// MFMAs of chunk kc issue.  Loads never branch: out-of-range rows or k read
// a zero page instead.
//
// Operand layouts.  The forward products use weights transposed once per
// call into the workspace (W1, W3 -> [E, h, d]; W2 -> [E, d, h]), so every
// operand of F1, F2, B1 and B3 has k contiguous: LDS rows are [position][k]
// with the eight 16-byte chunks of a row XOR-swizzled by the row index, so
// that fragment reads and row copies do not collide on banks.  The
// weight-gradient products B0 and B2 reduce over routes, so both of their
// operands have the M/N index contiguous: bf16 tiles stay [k][position] in
// LDS and MFMA fragments come from the transposing LDS read
// (ds_read_b64_tr_b16); float32 tiles are transposed in registers.
//
// Determinism: every output element has one writer.  The combine into y
// and the input gradient dx run as K ordered slot passes: pass k handles,
// for every token, its route in slot k (ascending expert id), so each token
// row is touched once per pass and the sum over slots is always taken in
// ascending k, in float32.

#include "moe_device.h"
#include "moe_internal.h"

#include <algorithm>
#include <type_traits>

namespace moe {

constexpr int NT = 512;                  // threads per workgroup
constexpr int TBM = 256;                 // output tile rows
constexpr int TBN = 256;                 // output tile columns (logical)
constexpr int ROWB = 128;                // bytes of k per LDS row per k-tile
constexpr int OPB = 256 * ROWB;          // one operand tile in LDS (32 KB)
constexpr int STAGE = 2 * OPB;           // A + B; two stages (128 KB)
constexpr int MT = 4, NTL = 2;           // MFMA 32x32 tiles per wavefront (M, N)

template <typename T> struct Traits;
template <> struct Traits<bf16_t> {
  static constexpr int ES = 2, VEC = 8, KT = 64;
};
template <> struct Traits<float> {
  static constexpr int ES = 4, VEC = 4, KT = 32;
};

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS row `row`.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  // Workgroups are handed out round-robin over the 8 XCDs; give each XCD a
  // contiguous run of logical tiles so neighbouring tiles share its L2.
  const int64_t per = nblocks >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// p advanced by a 32-bit byte offset (lets the compiler address with a
// scalar base and a 32-bit vector offset)
template <typename T>
__device__ __forceinline__ T* byte_off(T* p, uint32_t bytes) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + bytes);
}

__device__ __forceinline__ uint4 sel16(bool ok, uint4 v) {
  return ok ? v : make_uint4(0, 0, 0, 0);
}

// ------------------------------------------------------------------ loaders

typedef __attribute__((address_space(3))) char lds_char_t;

// 16 bytes per lane straight from global memory into LDS: lane i of the
// wavefront lands at lds_base + 16 i (lds_base is wavefront-uniform; it goes
// in M0, declared clobbered so the compiler keeps no value of its own there
// across the copy).  Written
// as inline assembly so that the compiler does not track these copies.
// Tracked, it must prove that a copy cannot write the LDS a fragment read is
// about to read, or else wait for every copy in flight before the read; that
// proof depends on how it happens to lower the stage addresses, and when it
// fails the copies and the MFMAs run back to back.  Every wait for the
// copies is explicit in the main loop.
// (M0 is a register the compiler reserves; clang warns that it does not
// track the liveness of reserved registers across inline assembly.  The
// clobber still records the write for the passes that look for one, and the
// gfx950 assembly is checked for other M0 users.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds(const void* g, char* lds_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_t*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 256 rows with k contiguous in memory, copied straight into LDS.  Element k
// of a row is at its start + k (k < ksplit) or start + delta + (k - ksplit)
// (k >= ksplit): the second source has the same row layout at a fixed byte
// distance.  Wavefront w fills rows w*32 .. w*32+31 with four 1 KB loads; in
// load j lane l writes
// LDS row w*32 + 8 j + (l >> 3), physical chunk l & 7, so it fetches the
// logical chunk (l & 7) ^ swizzle(row) of that row.  Absent rows and k
// beyond klen read the zero page instead.
template <typename T>
struct KLoaderD {
  static constexpr bool kDirect = true;
  const char* rp[4];      // row start (absent row: nullptr)
  int c0;                 // logical chunk fetched in load 0 (load j: c0 ^ j)
  const char* zero;       // 16 zero bytes
  int64_t delta;
  int ksplit, klen;

  __device__ static __forceinline__ int row_of(int j) {
    return (threadIdx.x >> 6) * 32 + 8 * j + ((threadIdx.x & 63) >> 3);
  }
  // Row r = 32 w + 8 j + (l >> 3) has swizzle (r ^ (r >> 3)) & 7 =
  // (l >> 3) ^ (4 (w & 1) + j) for j < 4, so load j fetches chunk c0 ^ j.
  __device__ __forceinline__ void init_chunks() {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    c0 = (l & 7) ^ (l >> 3) ^ ((w & 1) << 2);
  }
  __device__ __forceinline__ void issue(int kt, char* lds) const {
    constexpr int ES = Traits<T>::ES, VEC = Traits<T>::VEC, KT = Traits<T>::KT;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kt * KT + (c0 ^ j) * VEC;
      const bool ok = rp[j] != nullptr && k < klen;
      const char* g = k < ksplit ? rp[j] + (int64_t)k * ES : rp[j] + delta + (int64_t)(k - ksplit) * ES;
      load_to_lds(ok ? g : zero, lds + (w * 32 + 8 * j) * ROWB);
    }
  }
};

// Row pointers of a KLoaderD: LDS row r of the tile is list entry rb + r
// (identity list when list == nullptr), optionally mapped through `gather`;
// row index idx lives at base + idx * row_elems.
template <typename T>
__device__ __forceinline__ void kloaderd_rows(KLoaderD<T>& la, const T* base, const int32_t* list,
                                              const int32_t* gather, int rb, int re,
                                              int64_t row_elems, const char* zero) {
  la.zero = zero;
  la.init_chunks();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int li = rb + KLoaderD<T>::row_of(j);
    const char* p = nullptr;
    if (li < re) {
      int64_t idx = list != nullptr ? (int64_t)list[li] : (int64_t)li;
      if (gather != nullptr) idx = gather[idx];
      p = reinterpret_cast<const char*>(base + idx * row_elems);
    }
    la.rp[j] = p;
  }
}

// float32 operand of the weight-gradient products: 256 M/N positions with
// that index contiguous in memory, k indexing rows, transposed in registers
// on its way into the [position][k] LDS tile.  Row r(k) = ridx ? ridx[k] :
// rbase + k; the thread's 16-byte vector for k-row k is at col + r(k) * ld.
// Thread t owns positions (t >> 3) * 4 .. +4 and k-rows (t & 7) * 4 + i,
// i < 4 (a whole chunk); it writes 4 rows x 16 B.  Odd position groups write
// their rows in pair-swapped order so that consecutive lanes cover both row
// parities of an LDS cycle.  (bf16 uses TLoaderD.)
template <typename T>
struct MNLoader {
  static constexpr bool kDirect = false;
  const char* col;
  bool colok;
  int64_t ld;
  const int32_t* ridx;
  int64_t rbase;
  int klen;
  int64_t rnext[4];
  uint4 reg[4];

  __device__ static __forceinline__ int pos0();     // first position of the thread
  __device__ static __forceinline__ int krow0();    // first k-row of the thread in a tile

  // Positions first_pos + pos0() .. of `base` (an array with `limit`
  // positions per row and ld bytes between rows).
  __device__ __forceinline__ void setup(const char* base, int first_pos, int limit, int64_t ld_,
                                        const int32_t* ridx_, int64_t rbase_, int klen_) {
    constexpr int ES = Traits<T>::ES;
    const int p = first_pos + pos0();
    colok = p < limit;
    col = base + (int64_t)(colok ? p : 0) * ES;
    ld = ld_;
    ridx = ridx_;
    rbase = rbase_;
    klen = klen_;
    prime();
  }
  // Row indices of k-tile kt (gathered rows: loaded one k-tile ahead so that
  // the index load never sits in front of the data load).
  __device__ __forceinline__ void rows_of(int kt, int64_t (&rr)[4]) const {
    constexpr int KT = Traits<T>::KT;
    const int k0 = kt * KT + krow0();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + i;
      const bool in = colok && k < klen;  // the index array is never read past klen
      rr[i] = ridx != nullptr ? (in ? (int64_t)ridx[k] : 0) : rbase + (in ? k : 0);
    }
  }
  __device__ __forceinline__ void prime() { rows_of(0, rnext); }
  __device__ __forceinline__ void fetch(int kt) {
    constexpr int KT = Traits<T>::KT;
    const int k0 = kt * KT + krow0();
    int64_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = rnext[i];
    rows_of(kt + 1, rnext);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = colok && k0 + i < klen;
      reg[i] = sel16(ok, *reinterpret_cast<const uint4*>(col + r[i] * ld));
    }
  }
  __device__ __forceinline__ void store(char* lds) const;
};

template <>
__device__ __forceinline__ int MNLoader<float>::pos0() { return (threadIdx.x >> 3) * 4; }
template <>
__device__ __forceinline__ int MNLoader<float>::krow0() { return (threadIdx.x & 7) * 4; }

template <>
__device__ __forceinline__ void MNLoader<float>::store(char* lds) const {
  const int c = threadIdx.x & 7;
  const int n0 = pos0(), odd = (threadIdx.x >> 3) & 1;
  const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&reg[0]);
  const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&reg[1]);
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&reg[2]);
  const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&reg[3]);
  uint4 out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = make_uint4(q0[j], q1[j], q2[j], q3[j]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 v = odd ? out[j ^ 1] : out[j];
    *reinterpret_cast<uint4*>(lds + lds_off(n0 + (j ^ odd), c)) = v;
  }
}

// bf16 operand tile kept as it lies in memory: 64 k-rows x 256 positions
// (512 bytes per k-row).  MFMA fragments are read with the transposing LDS
// read (ds_read_b64_tr_b16), so no register transpose is needed.  The 32
// chunks of a k-row are XOR-swizzled by 4 * (k & 3), so that the four k-rows
// read together by a 16-lane group of the transposing read fall on
// different banks.
__device__ __forceinline__ int tlds_off(int k, int chunk) {
  return k * 512 + ((chunk ^ ((k & 3) << 2)) << 4);
}

// Loader of such a tile straight into LDS.  Wavefront w
// fills k-rows w*8 .. w*8+7 with four 1 KB loads; in load j lane l writes
// k-row w*8 + 2 j + (l >> 5), physical chunk l & 31, so it fetches logical
// chunk (l & 31) ^ (4 (k & 3)) = positions 8 c .. 8 c + 7.
struct TLoaderD {
  static constexpr bool kDirect = true;
  const char* col[4];     // position column of load j (row 0); absent: nullptr
  int64_t ld;
  const int32_t* ridx;
  int64_t rbase;
  int klen;
  const char* zero;
  int32_t rnext[4];       // row indices of the next k-tile (as loaded)

  __device__ static __forceinline__ int krow(int j) {
    return (threadIdx.x >> 6) * 8 + 2 * j + ((threadIdx.x & 63) >> 5);
  }
  __device__ static __forceinline__ int lpos(int j) {   // logical position of load j
    return (((threadIdx.x & 31) ^ ((krow(j) & 3) << 2))) * 8;
  }
  // Positions of the tile come from b0 (and, for dual tiles, b1 by the
  // interleave of dual_src / dual_col) starting at first_pos; `limit`
  // positions per row, ld bytes between rows.
  template <bool DUALCOL>
  __device__ __forceinline__ void setup(const char* b0, const char* b1, int first_pos, int limit,
                                        int64_t ld_, const int32_t* ridx_, int64_t rbase_,
                                        int klen_, const char* zero_);
  // The index array is never read past klen (a k-row past it reads entry 0
  // and copies the zero page instead).  The loaded value is used only by the
  // next k-tile's copies, so nothing waits for it here.
  __device__ __forceinline__ void rows_of(int kt, int32_t (&rr)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kt * 64 + krow(j);
      const bool in = k < klen;
      rr[j] = ridx != nullptr ? ridx[in ? k : 0] : (int32_t)rbase + (in ? k : 0);
    }
  }
  __device__ __forceinline__ void issue(int kt, char* lds) {
    int32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = rnext[j];
    rows_of(kt + 1, rnext);
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = col[j] != nullptr && kt * 64 + krow(j) < klen;
      const char* g = col[j] + r[j] * ld;
      load_to_lds(ok ? g : zero, lds + (w * 8 + 2 * j) * 512);
    }
  }
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Fragment of 32 positions p0 .. p0+31 and k = kbase .. kbase+15 from a
// TLoaderD tile: lane l gets position p0 + (l & 31) and the 8 k values
// kbase + 8 (l >> 5) + 0..7, from two transposing reads of 4 k-rows each.
// (Within a 16-lane group the read hands lane i element i & 3 of the
// 8-byte chunk addressed by lane 4 m + (i >> 2), for m = 0..3.)
__device__ __forceinline__ uint4 tr_fragment(const char* tile, int p0, int kbase) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  const int pos = p0 + 16 * (g & 1) + 4 * (i & 3);
  const int k0 = kbase + 8 * (g >> 1) + (i >> 2);
  const int cb = ((pos >> 3) & 31), half = (pos & 7) * 2;
  typedef __attribute__((address_space(3))) v4i16_t lds_v4;
  const lds_v4* a0 = reinterpret_cast<const lds_v4*>(
      (__attribute__((address_space(3))) const char*)(tile + tlds_off(k0, cb) + half));
  const lds_v4* a1 = reinterpret_cast<const lds_v4*>(
      (__attribute__((address_space(3))) const char*)(tile + tlds_off(k0 + 4, cb) + half));
  const v4i16_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4*>(a0));
  const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4*>(a1));
  const uint2 u0 = __builtin_bit_cast(uint2, x0);
  const uint2 u1 = __builtin_bit_cast(uint2, x1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

// ------------------------------------------------------------------ MFMA

template <typename T>
__device__ __forceinline__ f32x16_t mfma_k8(uint4 a, uint4 b, f32x16_t c);

template <>
__device__ __forceinline__ f32x16_t mfma_k8<bf16_t>(uint4 a, uint4 b, f32x16_t c) {
  // 8 bf16 per lane: one 32x32x16 product.
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16_t mfma_k8<float>(uint4 a, uint4 b, f32x16_t c) {
  // 4 float32 per lane: lanes 0-31 hold k = 0..3 and lanes 32-63 k = 4..7
  // of an 8-wide k group; product j pairs k = j with k = 4 + j.
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

struct Acc {
  f32x16_t c[MT][NTL];
};

// Wavefront w of the eight owns the 128 x 64 block (wave_m, wave_n) of the
// tile.  Wavefronts w and w + 4, which share a SIMD, differ in both their row
// half and their column half (w + 4 takes the other column half), so a tile
// whose last 128 rows or last 128 columns are padding still gives every SIMD
// one wavefront of MFMA work.
__device__ __forceinline__ int wave_m() { return (threadIdx.x >> 6) >> 2; }
__device__ __forceinline__ int wave_n() {
  const int w = threadIdx.x >> 6;
  return (w & 3) ^ ((w >> 2) << 1);
}

// MFMA fragments of two k-chunks (16 k each).  A k-tile's last chunk stays
// in slot 1 past the barrier that ends the tile: its MFMAs issue at the start
// of the next tile, after that tile's first fragment reads, so the LDS read
// latency after the barrier is covered.
struct Frags {
  uint4 a[2][MT], b[2][NTL];
};

template <typename T>
__device__ __forceinline__ void mma_chunk(const uint4 (&a)[MT], const uint4 (&b)[NTL], Acc& acc) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) acc.c[mt][nt] = mfma_k8<T>(a[mt], b[nt], acc.c[mt][nt]);
}

// fragments of k-chunk kc (k-tiles with k contiguous per LDS row)
__device__ __forceinline__ void read_chunk(const char* As, const char* Bs, int kc, uint4 (&a)[MT],
                                           uint4 (&b)[NTL]) {
  const int lane = threadIdx.x & 63;
  const int wm = wave_m(), wn = wave_n();
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    a[mt] = *reinterpret_cast<const uint4*>(As + lds_off(wm * 128 + mt * 32 + r, kc * 2 + g));
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt)
    b[nt] = *reinterpret_cast<const uint4*>(Bs + lds_off(wn * 64 + nt * 32 + r, kc * 2 + g));
}

// fragments of k-chunk kc from [k][position] tiles (transposing reads, bf16)
__device__ __forceinline__ void read_chunk_tr(const char* As, const char* Bs, int kc,
                                              uint4 (&a)[MT], uint4 (&b)[NTL]) {
  const int wm = wave_m(), wn = wave_n();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) a[mt] = tr_fragment(As, wm * 128 + mt * 32, kc * 16);
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) b[nt] = tr_fragment(Bs, wn * 64 + nt * 32, kc * 16);
}

// One k-tile of MFMAs.  pending: slot 1 holds the previous tile's last
// chunk.  On return slot 1 holds this tile's last chunk, not yet multiplied.
template <typename T, bool TR>
__device__ __forceinline__ void mma_ktile(const char* As, const char* Bs, Acc& acc, Frags& f,
                                          bool pending) {
  if constexpr (TR) read_chunk_tr(As, Bs, 0, f.a[0], f.b[0]);
  else read_chunk(As, Bs, 0, f.a[0], f.b[0]);
  // keep the reads above ahead of the MFMAs below
  __builtin_amdgcn_sched_barrier(0);
  if (pending) mma_chunk<T>(f.a[1], f.b[1], acc);
#pragma unroll
  for (int kc = 0; kc < 3; ++kc) {
    const int cb = kc & 1, nb = cb ^ 1;
    // fragments of k-chunk kc + 1 are read while the MFMAs of kc issue
    if constexpr (TR) read_chunk_tr(As, Bs, kc + 1, f.a[nb], f.b[nb]);
    else read_chunk(As, Bs, kc + 1, f.a[nb], f.b[nb]);
    __builtin_amdgcn_sched_barrier(0);
    mma_chunk<T>(f.a[cb], f.b[cb], acc);
  }
}

// Main loop over nk k-tiles; result in acc (zero when nk == 0).  TR: both
// operands are TLoaderD tiles read with the transposing LDS read.  smem
// holds two stages of [A | B] (128 KB).  Step kt sends out the copies of
// k-tile kt + 1 into the other stage, runs the MFMAs on stage kt, and waits
// for its copies before the barrier.  BFIRST: B's copies go out before A's
// (measured: the operand whose rows are gathered through an index array does
// best issued last).
// SKIP: `live` is false for a wavefront whose whole block lies in the
// padding of the tile; that wavefront runs a loop of its own that copies its
// share of the operands and meets every barrier, but reads no fragments and
// issues no MFMAs (its accumulators stay zero).
template <typename T, class LA, class LB, bool TR = false, bool BFIRST = false, bool SKIP = false>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, Acc& acc,
                                              bool live = true) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc.c[mt][nt][i] = 0.f;
  if (nk <= 0) return;
  constexpr bool DA = LA::kDirect, DB = LB::kDirect;
  if constexpr (SKIP) {
    static_assert(DA && DB, "copies-only loop for direct-to-LDS operands");
    if (__builtin_amdgcn_readfirstlane(live ? 1 : 0) == 0) {  // wave-uniform
      la.issue(0, smem);
      lb.issue(0, smem + OPB);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      for (int kt = 0; kt + 1 < nk; ++kt) {
        char* nxt = smem + ((kt + 1) & 1) * STAGE;
        if constexpr (BFIRST) lb.issue(kt + 1, nxt + OPB);
        la.issue(kt + 1, nxt);
        if constexpr (!BFIRST) lb.issue(kt + 1, nxt + OPB);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      __syncthreads();  // the live loop's last barrier
      return;
    }
  }
  if constexpr (DA) la.issue(0, smem); else { la.fetch(0); la.store(smem); }
  if constexpr (DB) lb.issue(0, smem + OPB); else { lb.fetch(0); lb.store(smem + OPB); }
  if constexpr (DA || DB) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  Frags f;
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      if constexpr (BFIRST) {
        if constexpr (DB) lb.issue(kt + 1, nxt + OPB); else lb.fetch(kt + 1);
      }
      if constexpr (DA) la.issue(kt + 1, nxt); else la.fetch(kt + 1);
      if constexpr (!BFIRST) {
        if constexpr (DB) lb.issue(kt + 1, nxt + OPB); else lb.fetch(kt + 1);
      }
    }
    mma_ktile<T, TR>(cur, cur + OPB, acc, f, kt > 0);
    if (more) {
      if constexpr (!DA) la.store(nxt);
      if constexpr (!DB) lb.store(nxt + OPB);
    }
    if constexpr (DA || DB) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  mma_chunk<T>(f.a[1], f.b[1], acc);
}

// Position of accumulator element i of MFMA tile (mt, nt) inside the
// 256 x 256 workgroup tile.
__device__ __forceinline__ int acc_row(int mt, int i) {
  const int lane = threadIdx.x & 63;
  return wave_m() * 128 + mt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
}
__device__ __forceinline__ int acc_col(int nt) {
  const int lane = threadIdx.x & 63;
  return wave_n() * 64 + nt * 32 + (lane & 31);
}
// Interleaved dual-B tiles (two matrices, 128 columns of each per tile):
// logical column lc -> matrix (lc >> 5) & 1, source column (lc >> 6) * 32 +
// (lc & 31).  A wavefront's accumulator tile 0 then holds matrix 0 and tile
// 1 holds matrix 1 at the same source column.
__device__ __forceinline__ int dual_src(int lc) { return (lc >> 5) & 1; }
__device__ __forceinline__ int dual_col(int lc) { return (lc >> 6) * 32 + (lc & 31); }

template <bool DUALCOL>
__device__ __forceinline__ void TLoaderD::setup(const char* b0, const char* b1, int first_pos,
                                                int limit, int64_t ld_, const int32_t* ridx_,
                                                int64_t rbase_, int klen_, const char* zero_) {
  ld = ld_;
  ridx = ridx_;
  rbase = rbase_;
  klen = klen_;
  zero = zero_;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lc = lpos(j);
    const int src = DUALCOL ? dual_src(lc) : 0;
    const int p = first_pos + (DUALCOL ? dual_col(lc) : lc);
    col[j] = p < limit ? (src == 0 ? b0 : b1) + (int64_t)p * 2 : nullptr;
  }
  rows_of(0, rnext);
}

template <typename T>
__device__ __forceinline__ float silu_of(float a);
// bf16 results: the hardware reciprocal (1 ulp) replaces the IEEE division,
// far below the bf16 rounding of everything these values feed.
template <>
__device__ __forceinline__ float silu_of<bf16_t>(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}
template <>
__device__ __forceinline__ float silu_of<float>(float a) { return a / (1.0f + expf(-a)); }
template <typename T>
__device__ __forceinline__ float sigm_of(float a);
template <>
__device__ __forceinline__ float sigm_of<bf16_t>(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}
template <>
__device__ __forceinline__ float sigm_of<float>(float a) { return 1.0f / (1.0f + expf(-a)); }

// ------------------------------------------------------------------ weights

// 16 bytes of a weight row as float32 (8 bf16 or 4 float32) and back.
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void load(const bf16_t* p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void store(bf16_t* p, const float (&v)[8]) {
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      q[k] = (uint32_t)f2bf(v[2 * k]) | ((uint32_t)f2bf(v[2 * k + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(q[0], q[1], q[2], q[3]);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// WT[e][c][r] = W[e][r][c] for an [E][R][C] tensor, 64 x 64 tiles through
// LDS, 16 bytes per global load and store (R and C are multiples of 8 and
// the tensors 16-byte aligned, so a 16-byte chunk never crosses a row end).
// A bf16 value passes through float32 and back unchanged.
template <typename T>
__global__ __launch_bounds__(256) void transpose_weights(const T* __restrict__ W,
                                                         T* __restrict__ WT, int R, int C) {
  constexpr int V = Vec16<T>::N;  // elements per chunk
  constexpr int CPR = 64 / V;     // chunks per 64-element tile row
  __shared__ float tile[64][65];
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const T* src = W + (int64_t)e * R * C;
  T* dst = WT + (int64_t)e * R * C;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, c = (i % CPR) * V;
    if (r0 + r < R && c0 + c < C) {
      float v[8];
      Vec16<T>::load(src + (int64_t)(r0 + r) * C + c0 + c, v);
#pragma unroll
      for (int u = 0; u < V; ++u) tile[r][c + u] = v[u];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int c = i / CPR, r = (i % CPR) * V;
    if (c0 + c < C && r0 + r < R) {
      float v[8];
#pragma unroll
      for (int u = 0; u < V; ++u) v[u] = tile[r + u][c];
      Vec16<T>::store(dst + (int64_t)(c0 + c) * R + r0 + r, v);
    }
  }
}

// ------------------------------------------------------------------ tiles

// Split each of G segment lists (seg[g*(E+1) + e] .. seg[g*(E+1) + e + 1])
// into row tiles of at most TBM rows.  desc[g][i] = {e, begin, end, 0} or
// {-1, 0, 0, 0} past the last tile.  E <= 1024: each thread counts the tiles
// of four consecutive experts.
constexpr int kMaxExperts = 1024;
__global__ __launch_bounds__(256) void tile_table(const int32_t* __restrict__ seg, int E,
                                                  int64_t max_tiles, int4* __restrict__ desc,
                                                  uint4* __restrict__ zero_page) {
  constexpr int EPT = kMaxExperts / 256;
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int scratch[4];
  if (zero_page != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 16)
    zero_page[threadIdx.x] = make_uint4(0, 0, 0, 0);
  const int grp = blockIdx.y;
  const int32_t* off = seg + (int64_t)grp * (E + 1);
  const int tid = threadIdx.x;
  int n[EPT], sum = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    n[j] = e < E ? (off[e + 1] - off[e] + TBM - 1) / TBM : 0;
    sum += n[j];
  }
  int tot;
  int ex = block256_incl_scan(sum, scratch, &tot) - sum;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    if (e < E) s_start[e] = ex;
    ex += n[j];
  }
  if (tid == 0) s_start[E] = tot;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  if (i >= max_tiles) return;
  int4 out = make_int4(-1, 0, 0, 0);
  if (i < tot) {
    int lo = 0, hi = E - 1;  // largest e with s_start[e] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int beg = off[lo] + (int)(i - s_start[lo]) * TBM;
    const int end = min(beg + TBM, off[lo + 1]);
    out = make_int4(lo, beg, end, 0);
  }
  desc[(int64_t)grp * max_tiles + i] = out;
}

// ------------------------------------------------------------------ slot lists
// Slot pass k processes, for every token, its slot-k route.  List k holds
// those route rows in ascending order (which groups them by expert), at
// list[k*L .. (k+1)*L); pe_off[k][e] are the expert boundaries inside it.

__global__ __launch_bounds__(256) void list_slots(const int32_t* __restrict__ tim,
                                                  const float* __restrict__ gates, int64_t R,
                                                  int K, uint8_t* __restrict__ slot_of,
                                                  float* __restrict__ gate_p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R) return;
  const int32_t p = tim[i];
  slot_of[p] = (uint8_t)(i % K);
  if (gate_p != nullptr) gate_p[p] = gates[i];
}

constexpr int LCH = 4096;  // routes per list chunk (16 per thread)

__device__ __forceinline__ void load_slots16(const uint8_t* slot_of, int64_t R, int64_t c,
                                             uint8_t s[16]) {
  const int64_t b = c * LCH + threadIdx.x * 16;
  if (b + 16 <= R) {
    const uint4 q = *reinterpret_cast<const uint4*>(slot_of + b);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = (uint8_t)(w[j >> 2] >> ((j & 3) * 8));
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = b + j < R ? slot_of[b + j] : (uint8_t)0xff;
  }
}

__global__ __launch_bounds__(256) void list_count(const uint8_t* __restrict__ slot_of, int64_t R,
                                                  int K, int C, int32_t* __restrict__ cnt) {
  __shared__ int scratch[4];
  uint8_t s[16];
  load_slots16(slot_of, R, blockIdx.x, s);
  for (int k = 0; k < K; ++k) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) n += s[j] == k;
    int tot;
    block256_incl_scan(n, scratch, &tot);
    if (threadIdx.x == 0) cnt[(int64_t)k * C + blockIdx.x] = tot;
  }
}

__global__ __launch_bounds__(256) void list_scatter(const uint8_t* __restrict__ slot_of,
                                                    int64_t R, int K, int C,
                                                    const int32_t* __restrict__ base,
                                                    int32_t* __restrict__ list) {
  __shared__ int scratch[4];
  uint8_t s[16];
  load_slots16(slot_of, R, blockIdx.x, s);
  const int64_t b = (int64_t)blockIdx.x * LCH + threadIdx.x * 16;
  for (int k = 0; k < K; ++k) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) n += s[j] == k;
    int tot;
    const int inc = block256_incl_scan(n, scratch, &tot);
    int pos = base[(int64_t)k * C + blockIdx.x] + inc - n;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (s[j] == k) list[pos++] = (int32_t)(b + j);
  }
}

__global__ __launch_bounds__(256) void list_bounds(const int32_t* __restrict__ list,
                                                   const int32_t* __restrict__ offsets, int64_t L,
                                                   int K, int E, int32_t* __restrict__ pe_off) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= K * (E + 1)) return;
  const int k = i / (E + 1), e = i % (E + 1);
  const int32_t* lst = list + (int64_t)k * L;
  const int32_t key = offsets[e];
  int64_t lo = 0, hi = L;  // first position with lst[pos] >= key
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (lst[mid] < key) lo = mid + 1; else hi = mid;
  }
  pe_off[i] = (int32_t)(k * L + lo);
}

// ------------------------------------------------------------------ G in pieces
// With G not kept (MOE_FLAG_RECOMPUTE_G) no [L*K, h] buffer exists: before
// each slot pass of the down-projection its L rows of G = SiLU(A) [* B] are
// formed from the checkpoint into an [L, h] buffer, and before dW2 the same
// buffer takes gate * G for one group of experts at a time (at most L
// routes).  G is computed in float32 from the bf16 (or float32) checkpoint
// and rounded once.

// 16 bytes of A and B (8 bf16 or 4 float32 each) -> 16 bytes of gate * G.
template <typename T>
__device__ __forceinline__ uint4 glu16(uint4 a, uint4 b, bool dual, float gate);
template <>
__device__ __forceinline__ uint4 glu16<bf16_t>(uint4 a, uint4 b, bool dual, float gate) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a0 = __uint_as_float(wa[k] << 16), a1 = __uint_as_float(wa[k] & 0xffff0000u);
    float g0 = silu_of<bf16_t>(a0), g1 = silu_of<bf16_t>(a1);
    if (dual) {
      g0 *= __uint_as_float(wb[k] << 16);
      g1 *= __uint_as_float(wb[k] & 0xffff0000u);
    }
    o[k] = (uint32_t)f2bf(gate * g0) | ((uint32_t)f2bf(gate * g1) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
template <>
__device__ __forceinline__ uint4 glu16<float>(uint4 a, uint4 b, bool dual, float gate) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float g = silu_of<float>(__uint_as_float(wa[k]));
    if (dual) g *= __uint_as_float(wb[k]);
    o[k] = __float_as_uint(gate * g);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// G rows formed ahead of a GEMM (MOE_FLAG_RECOMPUTE_G, one piece of at most
// L rows at a time), 16 bytes per thread:
//   list != nullptr: out[i] = SiLU(A[p]) [* B[p]], p = list[i], i < n
//                    (one slot pass's rows);
//   list == nullptr: out[i] = gate_p[p] * SiLU(A[p]) [* B[p]], p = r0 + i,
//                    r0 = offsets[chunk_e[c]], up to offsets[chunk_e[c + 1]]
//                    (the routes of expert group c, contiguous).
// Block (64, 4): a wavefront covers 64 consecutive chunks of one row; the
// grid walks the rows in steps (empty groups cost one short pass).
template <typename T, bool DUAL>
__global__ __launch_bounds__(256) void glu_rows(const T* __restrict__ A, const T* __restrict__ B,
                                                const int32_t* __restrict__ list,
                                                const float* __restrict__ gate_p,
                                                const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ chunk_e, int c,
                                                int64_t n, int h, T* __restrict__ out) {
  const int cpr = h * (int)sizeof(T) / 16;  // 16-byte chunks per row (h % 8 == 0)
  const int q = blockIdx.y * 64 + threadIdx.x;
  if (q >= cpr) return;
  int64_t r0 = 0;
  if (list == nullptr) {
    r0 = offsets[chunk_e[c]];
    n = offsets[chunk_e[c + 1]] - r0;
  }
  const int64_t rb = (int64_t)h * sizeof(T);  // row bytes
  // U rows per thread and sweep, every load out before the first store
  constexpr int U = 4;
  const int64_t S = (int64_t)gridDim.x * 4;
  for (int64_t i0 = (int64_t)blockIdx.x * 4 + threadIdx.y; i0 < n; i0 += S * U) {
    int64_t p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = min(i0 + u * S, n - 1);  // rows past n repeat row n - 1, not stored
      p[u] = list != nullptr ? (int64_t)list[i] : r0 + i;
    }
    uint4 a[U], b[U];
    float g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = p[u] * rb + q * 16;
      a[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(A) + o);
      b[u] = DUAL ? *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(B) + o) : a[u];
      g[u] = list != nullptr ? 1.0f : gate_p[p[u]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * S;
      if (i < n)
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(out) + i * rb + q * 16) =
            glu16<T>(a[u], b[u], DUAL, g[u]);
    }
  }
}

// Expert groups for dW2 under MOE_FLAG_RECOMPUTE_G: consecutive experts
// whose routes total at most cap = L, taken greedily from expert 0 (one
// expert alone never exceeds L).  Two neighbouring groups hold more than L
// routes together, so R = K L routes make at most 2K + 1 groups.
// chunk_e[g] is the first expert of group g; unused entries up to
// chunk_e[NC] are E (empty groups).
__global__ void glu_chunks(const int32_t* __restrict__ offsets, int E, int64_t cap, int NC,
                           int32_t* __restrict__ chunk_e) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int g = 0;
  chunk_e[0] = 0;
  int64_t start = offsets[0];
  for (int e = 0; e < E; ++e) {
    if ((int64_t)offsets[e + 1] - start > cap && g + 1 < NC) {
      chunk_e[++g] = e;
      start = offsets[e];
    }
  }
  for (int j = g + 1; j <= NC; ++j) chunk_e[j] = E;
}

// ------------------------------------------------------------------ kernels

struct RouteArgs {            // row tiles over routes or slot-pass lists
  const int4* tiles;
  int64_t ntiles;             // upper bound, rows of the grid
  int nN;                     // column tiles
  const char* zero;           // 16 zero bytes (workspace)
  int gm;                     // row tiles per window (1: row by row)
};

// Launch size of a route-major GEMM: whole windows, a multiple of the 8 XCDs.
static int64_t route_grid(const RouteArgs& ra) {
  const int64_t rows = (ra.ntiles + ra.gm - 1) / ra.gm * ra.gm;
  return (rows * ra.nN + 7) / 8 * 8;
}

// Tile coordinates of a route-major GEMM workgroup; false if it has no work.
// Each XCD takes a contiguous run of logical tiles (its own L2).  Inside a
// run, windows of gm row tiles are swept column tile by column tile, the
// row tile running fastest: with gm = 4 the 32 workgroups an XCD runs at
// once share four row tiles of A and eight column tiles of B, instead of
// three and eleven row by row for a dual tile of h = 1408 (eleven column
// tiles).
__device__ __forceinline__ bool route_tile(const RouteArgs& ra, int4& ds, int& ntile) {
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t wsz = (int64_t)ra.gm * ra.nN;
  const int64_t win = lid / wsz, r = lid % wsz;
  const int64_t mtile = win * ra.gm + r % ra.gm;
  ntile = (int)(r / ra.gm);
  if (mtile >= ra.ntiles) return false;
  ds = ra.tiles[mtile];
  return ds.x >= 0;
}

// ------------------------------------------------------------------ staged epilogues
// The epilogues below pass the accumulator tile through LDS a quarter at a
// time: MFMA row block q of both wavefront rows (tile rows 32q .. 32q + 31
// and 128 + 32q .. 128 + 32q + 31) as [64][256] float32 (64 KB), alternating
// between the two halves of the LDS.  LDS row r of quarter q is tile row
// (r / 32) * 128 + 32 q + r % 32.  Each thread then owns whole chunks of a
// row, so global loads and stores are 16 bytes per lane.

// MFMA row block qq of every wavefront -> LDS rows [64][256] f32 (buffer sb)
__device__ __forceinline__ void park_quarter(const Acc& acc, float* sb, int qq) {
  const int lane = threadIdx.x & 63;
  // this lane's first element; the others sit at constant offsets from it
  float* base = sb + (wave_m() * 32 + (lane >> 5) * 4) * 256 + acc_col(0);
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      base[((i >> 2) * 8 + (i & 3)) * 256 + nt * 32] = acc.c[qq][nt][i];
}

__device__ __forceinline__ int quarter_row(int qq, int r) { return (r >> 5) * 128 + qq * 32 + (r & 31); }

// Eight consecutive elements of a row, raw (as loaded) and as float32.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float v[8]) const {
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(q[k] << 16);
      v[2 * k + 1] = __uint_as_float(q[k] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float v[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  uint32_t q[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) q[k] = (uint32_t)f2bf(v[2 * k]) | ((uint32_t)f2bf(v[2 * k + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(q[0], q[1], q[2], q[3]);
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// eight float32 from LDS (16-byte aligned)
__device__ __forceinline__ void lds8(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// F1: [A | B] = X W1 [| X W3] with X gathered by expert_token_indices;
// epilogue writes A, B (checkpoint) and, with KEEPG, G = SiLU(A) [* B].
// W1T, W3T: [E, h, d] (transposed weights).
template <typename T, bool DUAL, bool KEEPG>
__global__ __launch_bounds__(NT, 1) void f1_gather_glu(RouteArgs ra, const T* __restrict__ x,
                                                       const T* __restrict__ W1T,
                                                       const T* __restrict__ W3T,
                                                       const int32_t* __restrict__ eti, int d,
                                                       int h, T* __restrict__ A,
                                                       T* __restrict__ B, T* __restrict__ G) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  constexpr int KT = Traits<T>::KT;
  int4 ds;
  int ntile;
  if (!route_tile(ra, ds, ntile)) return;
  // the tile descriptor is uniform: keep it in scalar registers
  const int e = __builtin_amdgcn_readfirstlane(ds.x);
  const int rb = __builtin_amdgcn_readfirstlane(ds.y), re = __builtin_amdgcn_readfirstlane(ds.z);
  const int n0 = ntile * (DUAL ? 128 : 256);

  KLoaderD<T> la;
  kloaderd_rows<T>(la, x, nullptr, eti, rb, re, d, ra.zero);
  la.delta = 0;
  la.ksplit = la.klen = d;
  KLoaderD<T> lb;
  lb.zero = ra.zero;
  lb.init_chunks();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lr = KLoaderD<T>::row_of(j);
    const int src = DUAL ? dual_src(lr) : 0;
    const int sc = n0 + (DUAL ? dual_col(lr) : lr);
    lb.rp[j] = sc < h ? reinterpret_cast<const char*>((src == 0 ? W1T : W3T) + ((int64_t)e * h + sc) * d)
                      : nullptr;
  }
  lb.delta = 0;
  lb.ksplit = lb.klen = d;
  Acc acc;
  gemm_mainloop<T>(la, lb, (d + KT - 1) / KT, smem, acc);

  // Stores address a scalar tile base plus a 32-bit byte offset.  A lane's
  // column and its row inside each group of four are fixed; the rest of the
  // row is uniform, so each row adds one scalar term to a fixed lane offset.
  // Full tiles (every tile of an expert segment but its last) skip the row
  // bound check.
  const int64_t tb = (int64_t)rb * h;
  T* At = A + tb;
  T* Bt = DUAL ? B + tb : nullptr;
  T* Gt = G + tb;
  const int lane = threadIdx.x & 63;
  const int wm = __builtin_amdgcn_readfirstlane(wave_m());
  const int nrows = re - rb;
  const int lrow = (lane >> 5) * 4;
  auto store_rows = [&](auto check) {
    constexpr bool CHECK = decltype(check)::value;
    if (DUAL) {
      const int c = n0 + dual_col(acc_col(0));
      if (c >= h) return;
      const uint32_t vo = (uint32_t)(lrow * h + c) * (uint32_t)sizeof(T);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ru = wm * 128 + mt * 32 + (i >> 2) * 8 + (i & 3);  // uniform
          if (CHECK && ru + lrow >= nrows) continue;
          const uint32_t o = vo + (uint32_t)(ru * h) * (uint32_t)sizeof(T);
          const float a = acc.c[mt][0][i], b = acc.c[mt][1][i];
          Elem<T>::store(byte_off(At, o), a);
          Elem<T>::store(byte_off(Bt, o), b);
          if (KEEPG) Elem<T>::store(byte_off(Gt, o), silu_of<T>(a) * b);
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const int c = n0 + acc_col(nt);
        if (c >= h) continue;
        const uint32_t vo = (uint32_t)(lrow * h + c) * (uint32_t)sizeof(T);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ru = wm * 128 + mt * 32 + (i >> 2) * 8 + (i & 3);
            if (CHECK && ru + lrow >= nrows) continue;
            const uint32_t o = vo + (uint32_t)(ru * h) * (uint32_t)sizeof(T);
            const float a = acc.c[mt][nt][i];
            Elem<T>::store(byte_off(At, o), a);
            if (KEEPG) Elem<T>::store(byte_off(Gt, o), silu_of<T>(a));
          }
        }
      }
    }
  };
  if (nrows >= 256)
    store_rows(std::false_type{});
  else
    store_rows(std::true_type{});
}

// Slot-pass epilogue: out/acc row t = s_t[row] (-1: no row), scale s_g[row].
//   MODE 0: only pass (K == 1): out = v
//   MODE 1: first pass:  acc = v
//   MODE 2: middle pass: acc += v
//   MODE 3: last pass:   out = acc + v
// For float32 outputs `acc` is the output itself (modes 1/2 only).
//
// Staged quarter by quarter (see park_quarter): each thread owns eight
// 16-byte chunks (four columns) of a quarter, so a wavefront covers one 1 KB
// accumulator row.  Quarter q is combined while quarter q + 1 is parked and
// the accumulator loads of quarter q + 2 are in flight.  d % 8 == 0 makes
// every chunk all in or all out.
constexpr int CCH = 8;  // chunks per thread per quarter: 64 rows x 64 chunks / NT

// Chunk j of a quarter, for wavefront w = threadIdx.x / 64: LDS row 8j + w,
// tile row cq(j) + 32 qq + w, columns 4 (threadIdx.x % 64) .. + 3.  Only w
// and the lane vary at run time, so every chunk's LDS address is a constant
// offset from one base.
__device__ __forceinline__ constexpr int cq(int j) { return (j >> 2) * 128 + (j & 3) * 8; }

template <int MODE, bool FULL>
__device__ __forceinline__ void combine_load(const int32_t* s_tw, int qq, int c, int d,
                                             const float* __restrict__ accb, float4 prev[CCH]) {
  if constexpr (MODE >= 2) {
#pragma unroll
    for (int j = 0; j < CCH; ++j) {
      const int t = s_tw[cq(j) + 32 * qq];
      const bool ok = FULL || (t >= 0 && c < d);
      // absent chunks read the (valid) first chunk and are never used
      const int64_t o = (int64_t)(ok ? t : 0) * d + (ok ? c : 0);
      prev[j] = *reinterpret_cast<const float4*>(accb + o);
    }
  }
}

template <typename T, int MODE, bool FULL>
__device__ __forceinline__ void combine_quarter(const float* sbw, const int32_t* s_tw,
                                                const float* s_gw, int qq, int c, int d,
                                                const float4 prev[CCH], T* __restrict__ out,
                                                float* __restrict__ accb) {
#pragma unroll
  for (int j = 0; j < CCH; ++j) {
    const int t = s_tw[cq(j) + 32 * qq];
    if (!FULL && (t < 0 || c >= d)) continue;
    const float g = s_gw[cq(j) + 32 * qq];
    const float4 a = *reinterpret_cast<const float4*>(sbw + j * 8 * 256);
    float4 v = make_float4(g * a.x, g * a.y, g * a.z, g * a.w);
    if constexpr (MODE >= 2)
      v = make_float4(prev[j].x + v.x, prev[j].y + v.y, prev[j].z + v.z, prev[j].w + v.w);
    const int64_t o = (int64_t)t * d + c;
    if constexpr (MODE == 1 || MODE == 2) {
      *reinterpret_cast<float4*>(accb + o) = v;
    } else if constexpr (std::is_same<T, float>::value) {
      *reinterpret_cast<float4*>(out + o) = v;
    } else {
      const uint2 w = make_uint2((uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16),
                                 (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16));
      *reinterpret_cast<uint2*>(out + o) = w;
    }
  }
}

// Called after the main loop's final barrier (LDS free, s_t / s_g visible).
// FULL: every row of the tile is present and every column is inside d, so
// no store is conditional.  (The compiler cannot count a store that a branch
// may skip; with such stores between the accumulator loads, its waits for
// the later loads also wait for earlier stores to complete.)
template <typename T, int MODE, bool FULL>
__device__ __forceinline__ void combine_epilogue(const Acc& acc, char* smem, const int32_t* s_t,
                                                 const float* s_g, int n0, int d,
                                                 T* __restrict__ out, float* __restrict__ accb) {
  const int w = threadIdx.x >> 6, cl = (threadIdx.x & 63) * 4;
  const int c = n0 + cl;
  float* sb[2] = {reinterpret_cast<float*>(smem), reinterpret_cast<float*>(smem + STAGE)};
  const int32_t* s_tw = s_t + w;
  const float* s_gw = s_g + w;
  float4 p[2][CCH];
  combine_load<MODE, FULL>(s_tw, 0, c, d, accb, p[0]);
  park_quarter(acc, sb[0], 0);
  combine_load<MODE, FULL>(s_tw, 1, c, d, accb, p[1]);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    // buffer (q + 1) & 1 was last read before the previous barrier
    if (q + 1 < MT) park_quarter(acc, sb[(q + 1) & 1], q + 1);
    combine_quarter<T, MODE, FULL>(sb[q & 1] + w * 256 + cl, s_tw, s_gw, q, c, d, p[q & 1], out,
                                   accb);
    if (q + 2 < MT) combine_load<MODE, FULL>(s_tw, q + 2, c, d, accb, p[q & 1]);
    if (q + 1 < MT) __syncthreads();
  }
}

template <typename T, bool FULL>
__device__ __forceinline__ void combine_modes(const Acc& acc, char* smem, const int32_t* s_t,
                                              const float* s_g, int n0, int d, int mode,
                                              T* __restrict__ out, float* __restrict__ accb) {
  switch (mode) {
    case 0: combine_epilogue<T, 0, FULL>(acc, smem, s_t, s_g, n0, d, out, accb); break;
    case 1: combine_epilogue<T, 1, FULL>(acc, smem, s_t, s_g, n0, d, out, accb); break;
    case 2: combine_epilogue<T, 2, FULL>(acc, smem, s_t, s_g, n0, d, out, accb); break;
    default: combine_epilogue<T, 3, FULL>(acc, smem, s_t, s_g, n0, d, out, accb); break;
  }
}

// nrows: rows present in the tile (the rest of s_t is -1).
template <typename T>
__device__ __forceinline__ void combine_dispatch(const Acc& acc, char* smem, const int32_t* s_t,
                                                 const float* s_g, int nrows, int n0, int d,
                                                 int mode, T* __restrict__ out,
                                                 float* __restrict__ accb) {
  // uniform across the workgroup; made scalar so the choice is one branch
  if (__builtin_amdgcn_readfirstlane((nrows == TBM && n0 + 256 <= d) ? 1 : 0))
    combine_modes<T, true>(acc, smem, s_t, s_g, n0, d, mode, out, accb);
  else
    combine_modes<T, false>(acc, smem, s_t, s_g, n0, d, mode, out, accb);
}

// F2 (slot pass k): O = G W2_e for the pass's rows, y[t] (+)= gate * O.
// W2T: [E, d, h] (transposed weights).  GM = 0: G read from Gb, row list[li];
// GM = 3: Gb holds only this pass's rows, row li - pbase (list position
// relative to the pass).
template <typename T, int GM>
__global__ __launch_bounds__(NT, 1) void f2_down_combine(RouteArgs ra, const T* __restrict__ Gb,
                                                         const T* __restrict__ W2T,
                                                         const int32_t* __restrict__ list,
                                                         const int32_t* __restrict__ eti,
                                                         const float* __restrict__ gates, int K,
                                                         int k, int d, int h, int mode,
                                                         int64_t pbase, T* __restrict__ y,
                                                         float* __restrict__ yacc) {
  static_assert(GM == 0 || GM == 3, "G read from the full buffer or from the pass's piece");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ int32_t s_t[TBM];
  __shared__ float s_g[TBM];
  constexpr int KT = Traits<T>::KT;
  int4 ds;
  int ntile;
  if (!route_tile(ra, ds, ntile)) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * 256;
  if (threadIdx.x < TBM) {
    const int li = rb + threadIdx.x;
    int32_t t = -1;
    float g = 0.f;
    if (li < re) {
      t = eti[list[li]];
      g = gates[(int64_t)t * K + k];
    }
    s_t[threadIdx.x] = t;
    s_g[threadIdx.x] = g;
  }

  KLoaderD<T> lb;
  kloaderd_rows<T>(lb, W2T + (int64_t)e * d * h, nullptr, nullptr, n0, d, h, ra.zero);
  lb.delta = 0;
  lb.ksplit = lb.klen = h;
  Acc acc;
  KLoaderD<T> la;
  if constexpr (GM == 0)
    kloaderd_rows<T>(la, Gb, list, nullptr, rb, re, h, ra.zero);
  else
    kloaderd_rows<T>(la, Gb, nullptr, nullptr, (int)(rb - pbase), (int)(re - pbase), h, ra.zero);
  la.delta = 0;
  la.ksplit = la.klen = h;
  gemm_mainloop<T>(la, lb, (h + KT - 1) / KT, smem, acc);
  __syncthreads();
  combine_dispatch<T>(acc, smem, s_t, s_g, re - rb, n0, d, mode, y, yacc);
}

// B1 epilogue on 8-column chunks: dG = gate * acc; with s = sigmoid(A),
// SiLU(A) = A s and SiLU'(A) = s (1 + A (1 - s)): dA = dG [* B] * SiLU'(A)
// and dB = dG * SiLU(A) are written over A and B, Gs = gate * SiLU(A) [* B].
// bf16: the checkpoint loads of quarter q + 1 are in flight while quarter q
// is processed.  ROUTER: dgp[p * nN + ntile] = sum over the tile's columns
// of acc * SiLU(A) [* B]; a row's 32 chunk lanes are summed by a fixed
// butterfly, so the value does not depend on timing.  FULL: all rows present
// and all columns inside h, so no store sits under a branch (see
// combine_epilogue for why that matters to the waits on the loads).
template <typename T, bool DUAL, bool ROUTER, bool FULL, bool KEEPG>
__device__ __forceinline__ void b1_epilogue(const Acc& acc, char* smem, const float* s_g, int rb,
                                            int re, int n0, int h, int nN, int ntile,
                                            T* __restrict__ A, T* __restrict__ B,
                                            T* __restrict__ Gs, float* __restrict__ dgp) {
  constexpr int CPT = 4;                    // chunks per thread per quarter (32 per row)
  constexpr bool PF = sizeof(T) == 2;       // prefetch the next quarter
  constexpr int NB = PF ? 2 : 1;
  float* sb[2] = {reinterpret_cast<float*>(smem), reinterpret_cast<float*>(smem + STAGE)};
  const int ch = threadIdx.x & 31, r0 = threadIdx.x >> 5;  // rows r0 + 16 j
  const int c = n0 + ch * 8;
  Raw8<T> xa[NB][CPT], xb[NB][CPT];
  auto load = [&](int q, int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int p = rb + quarter_row(q, r0 + 16 * j);
      const bool ok = FULL || (p < re && c < h);
      // absent chunks read the (valid) first chunk and are never used
      const int64_t o = ok ? (int64_t)p * h + c : 0;
      xa[buf][j].load(A + o);
      if (DUAL) xb[buf][j].load(B + o);
    }
  };
  if (PF) load(0, 0);
  park_quarter(acc, sb[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  if (PF) load(1, NB - 1);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    // buffer (q + 1) & 1 was last read before the previous barrier
    if (q + 1 < MT) park_quarter(acc, sb[(q + 1) & 1], q + 1);
    if (!PF) load(q, 0);
    const int buf = PF ? (q & 1) : 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int r = r0 + 16 * j;
      const int row = quarter_row(q, r);
      const int p = rb + row;
      float rdot = 0.f;
      if (FULL || (p < re && c < h)) {
        const int64_t o = (int64_t)p * h + c;
        const float gp = s_g[row];
        float v[8], a[8], b[8], da[8], db[8], gs[8];
        lds8(sb[q & 1] + r * 256 + ch * 8, v);
        xa[buf][j].get(a);
        if (DUAL) xb[buf][j].get(b);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float dg = gp * v[k];
          const float sg = sigm_of<T>(a[k]);
          const float sl = a[k] * sg;
          const float ds_ = sg * (1.0f + a[k] * (1.0f - sg));
          if (DUAL) {
            da[k] = dg * b[k] * ds_;
            db[k] = dg * sl;
            gs[k] = gp * sl * b[k];
            if (ROUTER) rdot += v[k] * (sl * b[k]);
          } else {
            da[k] = dg * ds_;
            gs[k] = gp * sl;
            if (ROUTER) rdot += v[k] * sl;
          }
        }
        store8(A + o, da);
        if (DUAL) store8(B + o, db);
        if (KEEPG) store8(Gs + o, gs);
      }
      if (ROUTER) {
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) rdot += __shfl_xor(rdot, m);
        if (ch == 0 && p < re) dgp[(int64_t)p * nN + ntile] = rdot;
      }
    }
    if (PF && q + 2 < MT) load(q + 2, q & 1);
    if (q + 1 < MT) __syncthreads();
  }
}

// B1: dG = gate * (dy[t] W2_e^T) per route; epilogue recomputes SiLU from
// the checkpoint and writes dA, dB over A, B and Gs = gate * G.  ROUTER: it
// also leaves, for every route row p, the tile's share of the router
// gradient's <dy[t] W2_e^T, G[p]> (= <dy[t], O[p]>, O the route's un-gated
// output) in dgp[p * nN + ntile].
template <typename T, bool DUAL, bool ROUTER, bool KEEPG>
__global__ __launch_bounds__(NT, 1) void b1_dgrad_glu(RouteArgs ra, const T* __restrict__ dy,
                                                      const T* __restrict__ W2,
                                                      const int32_t* __restrict__ eti,
                                                      const float* __restrict__ gate_p, int d,
                                                      int h, T* __restrict__ A,
                                                      T* __restrict__ B, T* __restrict__ Gs,
                                                      float* __restrict__ dgp) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ float s_g[TBM];
  constexpr int KT = Traits<T>::KT;
  int4 ds;
  int ntile;
  if (!route_tile(ra, ds, ntile)) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * 256;
  if (threadIdx.x < TBM) {
    const int p = rb + threadIdx.x;
    s_g[threadIdx.x] = p < re ? gate_p[p] : 0.f;
  }

  KLoaderD<T> la;
  kloaderd_rows<T>(la, dy, nullptr, eti, rb, re, d, ra.zero);
  la.delta = 0;
  la.ksplit = la.klen = d;
  KLoaderD<T> lb;
  kloaderd_rows<T>(lb, W2 + (int64_t)e * h * d, nullptr, nullptr, n0, h, d, ra.zero);
  lb.delta = 0;
  lb.ksplit = lb.klen = d;
  // with h % 256 == 128 the last column tile's second column half is padding
  const bool live = n0 + wave_n() * 64 < h && rb + wave_m() * 128 < re;
  Acc acc;
  gemm_mainloop<T, KLoaderD<T>, KLoaderD<T>, false, false, true>(la, lb, (d + KT - 1) / KT, smem,
                                                                   acc, live);
  __syncthreads();

  if (__builtin_amdgcn_readfirstlane((re - rb == TBM && n0 + 256 <= h) ? 1 : 0))
    b1_epilogue<T, DUAL, ROUTER, true, KEEPG>(acc, smem, s_g, rb, re, n0, h, ra.nN, ntile, A, B, Gs,
                                              dgp);
  else
    b1_epilogue<T, DUAL, ROUTER, false, KEEPG>(acc, smem, s_g, rb, re, n0, h, ra.nN, ntile, A, B,
                                               Gs, dgp);
}

// Router gradient, one workgroup per TB tokens (TB * E <= 16384: 64 tokens
// up to 256 experts, fewer beyond).  Every thread first takes routes (t, k)
// of the block: dg_k = <dy[t], O[tim[t, k]]> is the sum of the route's
// partials in ascending tile order, parked at the token's row in LDS under
// its expert.  Then lane t of wavefront 0 forms the softmax backward over
// the selected logits, dz_k = g_k (dg_k - sum_j g_j dg_j), sum in ascending
// k, in place; then the workgroup writes the TB full rows of dlogits (zeros
// for experts not chosen).
constexpr int kRouterRows = 16384;  // floats of LDS at most: TB rows of E (dynamic, TB * E used)
__global__ __launch_bounds__(256) void router_grad(const int32_t* __restrict__ tei,
                                                   const int32_t* __restrict__ tim,
                                                   const float* __restrict__ gates,
                                                   const float* __restrict__ dgp, int nN,
                                                   int64_t L, int E, int K, int TB,
                                                   float* __restrict__ dz) {
  extern __shared__ float s_rows[];  // TB * E floats, sized at launch
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int nrow = (int)min<int64_t>(TB, L - t0);
  for (int i = threadIdx.x; i < nrow * E; i += 256) s_rows[i] = 0.f;
  __syncthreads();
  const int nr = nrow * K;  // routes of the block: rows t0 .. t0 + nrow of tim, tei
  for (int i = threadIdx.x; i < nr; i += 256) {
    const int64_t r = t0 * K + i;
    const float* q = dgp + (int64_t)tim[r] * nN;
    const int e = tei[r];
    float dg = 0.f;
    int j = 0;
    for (; j + 4 <= nN; j += 4) {  // four loads in flight, summed in order
      const float q0 = q[j], q1 = q[j + 1], q2 = q[j + 2], q3 = q[j + 3];
      dg += q0;
      dg += q1;
      dg += q2;
      dg += q3;
    }
    for (; j < nN; ++j) dg += q[j];
    s_rows[(i / K) * E + e] = dg;
  }
  __syncthreads();
  if (threadIdx.x < nrow) {
    const int64_t t = t0 + threadIdx.x;
    const int32_t* te = tei + t * K;
    const float* g = gates + t * K;
    float* row = s_rows + threadIdx.x * E;
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += g[k] * row[te[k]];
    for (int k = 0; k < K; ++k) row[te[k]] = g[k] * (row[te[k]] - sum);
  }
  __syncthreads();
  float* out = dz + t0 * E;
  for (int i = threadIdx.x; i < nrow * E; i += 256) out[i] = s_rows[i];
}

struct WeightArgs {           // weight-gradient tiles: E x nM x nN
  int E, nM, nN;
  const char* zero;           // 16 zero bytes (workspace)
};

// Weight-gradient tiles are taken in launch order, which deals the tiles of
// one expert round-robin over the XCDs: a tile's cost is its expert's route
// count, so giving each XCD a contiguous run of experts (as the route-major
// products do) would pile the heaviest experts onto one XCD when loads are
// skewed.  Inside an expert the faster-running tile index is the one whose
// count is a multiple of the 8 XCDs (N if both are), so that every tile an
// XCD receives from an expert shares that XCD's operand block on the other
// side (same M block, or same N block) and reads it from its own L2.
__device__ __forceinline__ bool weight_tile(const WeightArgs& wa, int& e, int& mi, int& ni) {
  const int64_t lid = blockIdx.x;
  const int64_t per_e = (int64_t)wa.nM * wa.nN;
  if (lid >= (int64_t)wa.E * per_e) return false;
  e = (int)(lid / per_e);
  const int rem = (int)(lid % per_e);
  const bool mfast = (wa.nN & 7) != 0 && (wa.nM & 7) == 0;
  mi = mfast ? rem % wa.nM : rem / wa.nN;
  ni = mfast ? rem / wa.nM : rem % wa.nN;
  return true;
}

// B0: dW2_e = Gs_e^T dy_e (reduction over the expert's routes, ascending).
// GM = 0: Gs = gate * G read from the buffer the dG kernel wrote; GM = 3:
// Gs holds only the routes of expert group c (experts chunk_e[c] ..
// chunk_e[c + 1] - 1, from route offsets[chunk_e[c]] on), formed from A, B
// before the dG kernel replaces them, and the other experts' workgroups
// return.
template <typename T, int GM>
__global__ __launch_bounds__(NT, 1) void b0_dw2(WeightArgs wa, const T* __restrict__ Gs,
                                                const T* __restrict__ dy,
                                                const int32_t* __restrict__ eti,
                                                const int32_t* __restrict__ offsets, int d, int h,
                                                const int32_t* __restrict__ chunk_e, int c,
                                                T* __restrict__ dW2) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  static_assert(GM == 0 || GM == 3, "gate * G from the full buffer or from a group's piece");
  constexpr int ES = Traits<T>::ES, KT = Traits<T>::KT;
  int e, mi, ni;
  if (!weight_tile(wa, e, mi, ni)) return;
  int gbase = 0;  // first route held in Gs
  if constexpr (GM == 3) {
    const int e0 = chunk_e[c], e1 = chunk_e[c + 1];
    if (e < e0 || e >= e1) return;
    gbase = offsets[e0];
  }
  const int m0 = mi * 256, n0 = ni * 256;
  const int o0 = offsets[e], n_e = offsets[e + 1] - o0;
  // with h % 256 == 128 the last M tile's second row half is padding
  const bool live = m0 + wave_m() * 128 < h && n0 + wave_n() * 64 < d;

  Acc acc;
  if constexpr (std::is_same<T, bf16_t>::value) {
    TLoaderD lb;
    lb.setup<false>(reinterpret_cast<const char*>(dy), nullptr, n0, d, (int64_t)d * ES, eti + o0,
                    0, n_e, wa.zero);
    TLoaderD la;
    la.setup<false>(reinterpret_cast<const char*>(Gs), nullptr, m0, h, (int64_t)h * ES, nullptr,
                    o0 - gbase, n_e, wa.zero);
    gemm_mainloop<T, TLoaderD, TLoaderD, true, false, true>(la, lb, (n_e + KT - 1) / KT, smem, acc,
                                                            live);
  } else {
    MNLoader<T> lb;
    lb.setup(reinterpret_cast<const char*>(dy), n0, d, (int64_t)d * ES, eti + o0, 0, n_e);
    MNLoader<T> la;
    la.setup(reinterpret_cast<const char*>(Gs), m0, h, (int64_t)h * ES, nullptr, o0 - gbase, n_e);
    gemm_mainloop<T>(la, lb, (n_e + KT - 1) / KT, smem, acc);
  }

  T* out = dW2 + (int64_t)e * h * d;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + acc_row(mt, i);
      if (m >= h) continue;
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const int c = n0 + acc_col(nt);
        if (c < d) Elem<T>::store(out + (int64_t)m * d + c, acc.c[mt][nt][i]);
      }
    }
}

// B2: dW1_e = X_e^T dA_e [, dW3_e = X_e^T dB_e], X gathered by
// expert_token_indices; both products share the X tile (interleaved columns).
template <typename T, bool DUAL>
__global__ __launch_bounds__(NT, 1) void b2_dw13(WeightArgs wa, const T* __restrict__ x,
                                                 const T* __restrict__ dA,
                                                 const T* __restrict__ dB,
                                                 const int32_t* __restrict__ eti,
                                                 const int32_t* __restrict__ offsets, int d,
                                                 int h, T* __restrict__ dW1,
                                                 T* __restrict__ dW3) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  constexpr int ES = Traits<T>::ES, KT = Traits<T>::KT;
  int e, mi, ni;
  if (!weight_tile(wa, e, mi, ni)) return;
  const int m0 = mi * 256, n0 = ni * (DUAL ? 128 : 256);
  const int o0 = offsets[e], n_e = offsets[e + 1] - o0;

  Acc acc;
  if constexpr (std::is_same<T, bf16_t>::value) {
    TLoaderD la, lb;
    la.setup<false>(reinterpret_cast<const char*>(x), nullptr, m0, d, (int64_t)d * ES, eti + o0, 0,
                    n_e, wa.zero);
    lb.setup<DUAL>(reinterpret_cast<const char*>(dA), reinterpret_cast<const char*>(dB), n0, h,
                   (int64_t)h * ES, nullptr, o0, n_e, wa.zero);
    // x rows are gathered: their copies go out last
    gemm_mainloop<T, TLoaderD, TLoaderD, true, true>(la, lb, (n_e + KT - 1) / KT, smem, acc);
  } else {
    MNLoader<T> la, lb;
    la.setup(reinterpret_cast<const char*>(x), m0, d, (int64_t)d * ES, eti + o0, 0, n_e);
    // Logical column lc of this thread's first position -> (matrix, source
    // column); setup() adds lc to first_pos, so pass n0 + source column - lc.
    const int lc = MNLoader<T>::pos0();
    const int src = DUAL ? dual_src(lc) : 0;
    const int sc = DUAL ? dual_col(lc) : lc;
    lb.setup(reinterpret_cast<const char*>(src == 0 ? dA : dB), n0 + sc - lc, h,
             (int64_t)h * ES, nullptr, o0, n_e);
    gemm_mainloop<T>(la, lb, (n_e + KT - 1) / KT, smem, acc);
  }

  T* o1 = dW1 + (int64_t)e * d * h;
  T* o3 = DUAL ? dW3 + (int64_t)e * d * h : nullptr;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + acc_row(mt, i);
      if (m >= d) continue;
      if (DUAL) {
        const int c = n0 + dual_col(acc_col(0));
        if (c < h) {
          Elem<T>::store(o1 + (int64_t)m * h + c, acc.c[mt][0][i]);
          Elem<T>::store(o3 + (int64_t)m * h + c, acc.c[mt][1][i]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
          const int c = n0 + acc_col(nt);
          if (c < h) Elem<T>::store(o1 + (int64_t)m * h + c, acc.c[mt][nt][i]);
        }
      }
    }
}

// B3 (slot pass k): dX = [dA | dB] [W1_e | W3_e]^T for the pass's rows,
// dx[t] (+)= dX.  One GEMM over the concatenated 2h.
template <typename T, bool DUAL>
__global__ __launch_bounds__(NT, 1) void b3_dx(RouteArgs ra, const T* __restrict__ dA,
                                               const T* __restrict__ dB,
                                               const T* __restrict__ W1,
                                               const T* __restrict__ W3,
                                               const int32_t* __restrict__ list,
                                               const int32_t* __restrict__ eti, int d, int h,
                                               int mode, T* __restrict__ dx,
                                               float* __restrict__ dxacc) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ int32_t s_t[TBM];
  __shared__ float s_g[TBM];
  constexpr int KT = Traits<T>::KT;
  int4 ds;
  int ntile;
  if (!route_tile(ra, ds, ntile)) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * 256;
  const int klen = DUAL ? 2 * h : h;
  if (threadIdx.x < TBM) {
    const int li = rb + threadIdx.x;
    s_t[threadIdx.x] = li < re ? eti[list[li]] : -1;
    s_g[threadIdx.x] = 1.0f;
  }

  KLoaderD<T> la;
  kloaderd_rows<T>(la, dA, list, nullptr, rb, re, h, ra.zero);
  la.delta = DUAL ? (reinterpret_cast<const char*>(dB) - reinterpret_cast<const char*>(dA)) : 0;
  la.ksplit = h;
  la.klen = klen;
  KLoaderD<T> lb;
  kloaderd_rows<T>(lb, W1 + (int64_t)e * d * h, nullptr, nullptr, n0, d, h, ra.zero);
  lb.delta = DUAL ? (reinterpret_cast<const char*>(W3) - reinterpret_cast<const char*>(W1)) : 0;
  lb.ksplit = h;
  lb.klen = klen;
  Acc acc;
  gemm_mainloop<T>(la, lb, (klen + KT - 1) / KT, smem, acc);
  __syncthreads();
  combine_dispatch<T>(acc, smem, s_t, s_g, re - rb, n0, d, mode, dx, dxacc);
}

// ------------------------------------------------------------------ host

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

FfnPlan plan_ffn(const FfnDims& dm, bool backward) {
  FfnPlan p;
  const int es = dm.dtype == 1 ? 2 : 4;
  p.R = dm.L * dm.K;
  p.route_tiles = cdiv(p.R, TBM) + dm.E;
  p.pass_tiles = cdiv(dm.L, TBM) + dm.E;
  p.list_chunks = cdiv(p.R, LCH);
  const bool need_acc = dm.dtype == 1 && dm.K > 1;
  const size_t wbytes = (size_t)dm.E * dm.d * dm.h * es;
  size_t o = 0;
  // G (forward) or gate * G (backward) for all R routes; with recompute_g
  // one piece of at most L rows at a time (a slot pass's rows, or a group of
  // experts: an expert has at most one route per token)
  p.off_g = o;
  o = align_up(o + (size_t)(dm.recompute_g ? dm.L : p.R) * dm.h * es, 256);
  p.off_acc = o;    o = align_up(o + (need_acc ? (size_t)dm.L * dm.d * 4 : 0), 256);
  p.off_slot = o;   o = align_up(o + (size_t)p.R + 16, 256);
  p.off_list = o;   o = align_up(o + (size_t)p.R * 4, 256);
  p.off_cnt = o;    o = align_up(o + (size_t)dm.K * p.list_chunks * 4, 256);
  p.off_base = o;   o = align_up(o + (size_t)dm.K * p.list_chunks * 4, 256);
  p.off_peoff = o;  o = align_up(o + (size_t)dm.K * (dm.E + 1) * 4, 256);
  p.off_gatep = o;  o = align_up(o + (backward ? (size_t)p.R * 4 : 0), 256);
  // router gradient: per route, one partial <dG row, G row> per 256-column tile
  p.off_dgp = o;    o = align_up(o + (backward ? (size_t)p.R * cdiv(dm.h, 256) * 4 : 0), 256);
  p.off_tiles_route = o; o = align_up(o + (size_t)p.route_tiles * 16, 256);
  p.off_tiles_pass = o;  o = align_up(o + (size_t)dm.K * p.pass_tiles * 16, 256);
  const int nW = backward ? 0 : (dm.act == 1 ? 3 : 2);   // W1T, W2T, (W3T)
  p.off_wt = o;     o = align_up(o + nW * wbytes, 256);
  p.off_zero = o;   o = align_up(o + 256, 256);
  p.n_chunk = dm.recompute_g && backward ? 2 * dm.K + 1 : 0;
  p.off_chunk = o;  o = align_up(o + (size_t)(p.n_chunk + 1) * 4, 256);
  p.bytes = o;
  return p;
}

struct Lists {
  int32_t* list;
  int32_t* pe_off;
  int4* tiles_route;
  int4* tiles_pass;
  uint4* zero;
};

static Lists build_lists(const FfnPlan& pl, const FfnDims& dm, const int32_t* offsets,
                         const int32_t* tim, const float* gates, float* gate_p, char* ws,
                         hipStream_t s) {
  Lists ls;
  uint8_t* slot_of = reinterpret_cast<uint8_t*>(ws + pl.off_slot);
  ls.list = reinterpret_cast<int32_t*>(ws + pl.off_list);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + pl.off_cnt);
  int32_t* base = reinterpret_cast<int32_t*>(ws + pl.off_base);
  ls.pe_off = reinterpret_cast<int32_t*>(ws + pl.off_peoff);
  ls.tiles_route = reinterpret_cast<int4*>(ws + pl.off_tiles_route);
  ls.tiles_pass = reinterpret_cast<int4*>(ws + pl.off_tiles_pass);
  ls.zero = reinterpret_cast<uint4*>(ws + pl.off_zero);
  const int C = (int)pl.list_chunks;
  {
    LaunchTimer lt("route_tiles", s);
    hipLaunchKernelGGL(tile_table, dim3((unsigned)cdiv(pl.route_tiles, 256), 1), dim3(256), 0, s,
                       offsets, dm.E, pl.route_tiles, ls.tiles_route, ls.zero);
  }
  {
    LaunchTimer lt("slot_lists", s);
    hipLaunchKernelGGL(list_slots, dim3((unsigned)cdiv(pl.R, 256)), dim3(256), 0, s, tim, gates,
                       pl.R, dm.K, slot_of, gate_p);
    hipLaunchKernelGGL(list_count, dim3(C), dim3(256), 0, s, slot_of, pl.R, dm.K, C, cnt);
    launch_seg_scan(cnt, dm.K, C, dm.L, base, nullptr, s);
    hipLaunchKernelGGL(list_scatter, dim3(C), dim3(256), 0, s, slot_of, pl.R, dm.K, C, base,
                       ls.list);
    hipLaunchKernelGGL(list_bounds, dim3((unsigned)cdiv((int64_t)dm.K * (dm.E + 1), 256)),
                       dim3(256), 0, s, ls.list, offsets, dm.L, dm.K, dm.E, ls.pe_off);
  }
  {
    LaunchTimer lt("pass_tiles", s);
    hipLaunchKernelGGL(tile_table, dim3((unsigned)cdiv(pl.pass_tiles, 256), dm.K), dim3(256), 0,
                       s, ls.pe_off, dm.E, pl.pass_tiles, ls.tiles_pass, (uint4*)nullptr);
  }
  return ls;
}

static int pass_mode(int K, int k, bool f32) {
  if (K == 1) return f32 ? 1 : 0;
  if (k == 0) return 1;
  if (k < K - 1) return 2;
  return f32 ? 2 : 3;
}

template <typename T>
static void transpose_w(const T* W, T* WT, int E, int R, int C, hipStream_t s) {
  hipLaunchKernelGGL((transpose_weights<T>), dim3((unsigned)cdiv(C, 64), (unsigned)cdiv(R, 64), E),
                     dim3(256), 0, s, W, WT, R, C);
}

// G rows ahead of a GEMM (see glu_rows); nmax bounds the rows (n is read on
// the device for expert groups).
template <typename T>
static void glu_launch(bool dual, const T* A, const T* B, const int32_t* list,
                       const float* gate_p, const int32_t* offsets, const int32_t* chunk_e, int c,
                       int64_t nmax, int h, T* out, hipStream_t s) {
  const int cpr = h * (int)sizeof(T) / 16;
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(nmax, 16), 16384)),
                  (unsigned)cdiv(cpr, 64));
  if (dual)
    hipLaunchKernelGGL((glu_rows<T, true>), grid, dim3(64, 4), 0, s, A, B, list, gate_p, offsets,
                       chunk_e, c, nmax, h, out);
  else
    hipLaunchKernelGGL((glu_rows<T, false>), grid, dim3(64, 4), 0, s, A, B, list, gate_p, offsets,
                       chunk_e, c, nmax, h, out);
}

template <typename T>
static void forward_t(const FfnPlan& pl, const FfnDims& dm, const T* x, const T* W1, const T* W3,
                      const T* W2, const int32_t* eti, const int32_t* offsets, const int32_t* tim,
                      const float* gates, T* y, T* A, T* B, char* ws, hipStream_t s) {
  const bool f32 = sizeof(T) == 4;
  const bool dual = dm.act == 1;
  const size_t wel = (size_t)dm.E * dm.d * dm.h;
  T* W1T = reinterpret_cast<T*>(ws + pl.off_wt);
  T* W2T = W1T + wel;
  T* W3T = dual ? W2T + wel : W1T;
  {
    LaunchTimer lt("weight_transpose", s);
    transpose_w<T>(W1, W1T, dm.E, dm.d, dm.h, s);
    if (dual) transpose_w<T>(W3, W3T, dm.E, dm.d, dm.h, s);
    transpose_w<T>(W2, W2T, dm.E, dm.h, dm.d, s);
  }
  Lists ls = build_lists(pl, dm, offsets, tim, gates, nullptr, ws, s);
  T* G = reinterpret_cast<T*>(ws + pl.off_g);
  float* acc = f32 ? reinterpret_cast<float*>(y) : reinterpret_cast<float*>(ws + pl.off_acc);
  const bool keepg = !dm.recompute_g;
  {
    LaunchTimer lt("ffn_f1_gather_glu", s);
    RouteArgs ra{ls.tiles_route, pl.route_tiles, (int)cdiv(dm.h, dual ? 128 : 256), (const char*)ls.zero, 4};
    const unsigned grid = (unsigned)route_grid(ra);
#define MOE_F1(DU, KG)                                                                          \
  hipLaunchKernelGGL((f1_gather_glu<T, DU, KG>), dim3(grid), dim3(NT), 0, s, ra, x, W1T, W3T, eti, \
                     dm.d, dm.h, A, B, G)
    if (dual) {
      if (keepg) MOE_F1(true, true); else MOE_F1(true, false);
    } else {
      if (keepg) MOE_F1(false, true); else MOE_F1(false, false);
    }
#undef MOE_F1
  }
  // G kept: F1 wrote it for every route.  Not kept: before each pass, the
  // pass's L rows of G are formed from A, B into the same buffer.
  const int gm = keepg ? 0 : 3;
  for (int k = 0; k < dm.K; ++k) {
    if (!keepg) {
      LaunchTimer lt("glu_transient", s);
      glu_launch<T>(dual, A, B, ls.list + (int64_t)k * dm.L, nullptr, nullptr, nullptr, 0, dm.L,
                    dm.h, G, s);
    }
    LaunchTimer lt("ffn_f2_down_combine", s);
    RouteArgs ra{ls.tiles_pass + (int64_t)k * pl.pass_tiles, pl.pass_tiles, (int)cdiv(dm.d, 256), (const char*)ls.zero, 1};
    const unsigned grid = (unsigned)route_grid(ra);
#define MOE_F2(GMV)                                                                             \
  hipLaunchKernelGGL((f2_down_combine<T, GMV>), dim3(grid), dim3(NT), 0, s, ra, G, W2T,           \
                     ls.list, eti, gates, dm.K, k, dm.d, dm.h, pass_mode(dm.K, k, f32),           \
                     (int64_t)k * dm.L, y, acc)
    if (gm == 0) MOE_F2(0); else MOE_F2(3);
#undef MOE_F2
  }
}

template <typename T>
static void backward_t(const FfnPlan& pl, const FfnDims& dm, const T* dy, const T* x, const T* W1,
                       const T* W3, const T* W2, const int32_t* eti, const int32_t* offsets,
                       const int32_t* tim, const float* gates, T* A, T* B, T* dx, T* dW1, T* dW3,
                       T* dW2, const int32_t* tei, float* dlogits, char* ws, hipStream_t s) {
  const bool f32 = sizeof(T) == 4;
  const bool dual = dm.act == 1;
  float* gate_p = reinterpret_cast<float*>(ws + pl.off_gatep);
  Lists ls = build_lists(pl, dm, offsets, tim, gates, gate_p, ws, s);
  T* Gs = reinterpret_cast<T*>(ws + pl.off_g);
  int32_t* chunk_e = reinterpret_cast<int32_t*>(ws + pl.off_chunk);
  float* acc = f32 ? reinterpret_cast<float*>(dx) : reinterpret_cast<float*>(ws + pl.off_acc);
  float* dgp = dlogits != nullptr ? reinterpret_cast<float*>(ws + pl.off_dgp) : nullptr;
  const int nNh = (int)cdiv(dm.h, 256);
  const bool keepg = !dm.recompute_g;
  // dW2 needs gate * G: from the dG kernel's buffer (after it), or, not kept,
  // formed from A, B (before the dG kernel writes dA, dB over them) one
  // expert group of at most L routes at a time into the same buffer
  auto dw2 = [&]() {
    WeightArgs wa{dm.E, (int)cdiv(dm.h, 256), (int)cdiv(dm.d, 256), (const char*)ls.zero};
    const int64_t n = (int64_t)dm.E * wa.nM * wa.nN;
#define MOE_B0(GMV, C)                                                                          \
  hipLaunchKernelGGL((b0_dw2<T, GMV>), dim3((unsigned)round8(n)), dim3(NT), 0, s, wa, Gs, dy, eti, \
                     offsets, dm.d, dm.h, chunk_e, C, dW2)
    if (keepg) {
      LaunchTimer lt("ffn_b0_dw2", s);
      MOE_B0(0, 0);
      return;
    }
    {
      LaunchTimer lt("glu_transient", s);
      hipLaunchKernelGGL(glu_chunks, dim3(1), dim3(64), 0, s, offsets, dm.E, dm.L, pl.n_chunk,
                         chunk_e);
    }
    for (int c = 0; c < pl.n_chunk; ++c) {
      {
        LaunchTimer lt("glu_transient", s);
        glu_launch<T>(dual, A, B, nullptr, gate_p, offsets, chunk_e, c, dm.L, dm.h, Gs, s);
      }
      LaunchTimer lt("ffn_b0_dw2", s);
      MOE_B0(3, c);
    }
#undef MOE_B0
  };
  if (!keepg) dw2();
  {
    LaunchTimer lt("ffn_b1_dgrad_glu", s);
    RouteArgs ra{ls.tiles_route, pl.route_tiles, nNh, (const char*)ls.zero, 1};
    const unsigned grid = (unsigned)route_grid(ra);
#define MOE_B1(DU, RO, KG)                                                                      \
  hipLaunchKernelGGL((b1_dgrad_glu<T, DU, RO, KG>), dim3(grid), dim3(NT), 0, s, ra, dy, W2, eti,  \
                     gate_p, dm.d, dm.h, A, B, Gs, dgp)
#define MOE_B1K(DU, RO) \
  if (keepg) MOE_B1(DU, RO, true); else MOE_B1(DU, RO, false)
    if (dual) {
      if (dgp != nullptr) MOE_B1K(true, true);
      else MOE_B1K(true, false);
    } else {
      if (dgp != nullptr) MOE_B1K(false, true);
      else MOE_B1K(false, false);
    }
#undef MOE_B1K
#undef MOE_B1
  }
  if (dlogits != nullptr) {
    LaunchTimer lt("router_grad", s);
    const int TB = std::min(64, kRouterRows / dm.E);
    hipLaunchKernelGGL(router_grad, dim3((unsigned)cdiv(dm.L, TB)), dim3(256),
                       (size_t)TB * dm.E * sizeof(float), s, tei, tim, gates, dgp, nNh, dm.L, dm.E,
                       dm.K, TB, dlogits);
  }
  if (keepg) dw2();
  {
    LaunchTimer lt("ffn_b2_dw13", s);
    WeightArgs wa{dm.E, (int)cdiv(dm.d, 256), (int)cdiv(dm.h, dual ? 128 : 256), (const char*)ls.zero};
    const int64_t n = (int64_t)dm.E * wa.nM * wa.nN;
    if (dual)
      hipLaunchKernelGGL((b2_dw13<T, true>), dim3((unsigned)round8(n)), dim3(NT), 0, s, wa, x, A,
                         B, eti, offsets, dm.d, dm.h, dW1, dW3);
    else
      hipLaunchKernelGGL((b2_dw13<T, false>), dim3((unsigned)round8(n)), dim3(NT), 0, s, wa, x, A,
                         B, eti, offsets, dm.d, dm.h, dW1, dW3);
  }
  for (int k = 0; k < dm.K; ++k) {
    LaunchTimer lt("ffn_b3_dx", s);
    RouteArgs ra{ls.tiles_pass + (int64_t)k * pl.pass_tiles, pl.pass_tiles, (int)cdiv(dm.d, 256), (const char*)ls.zero, 1};
    const unsigned grid = (unsigned)route_grid(ra);
    if (dual)
      hipLaunchKernelGGL((b3_dx<T, true>), dim3(grid), dim3(NT), 0, s, ra, A, B, W1, W3, ls.list,
                         eti, dm.d, dm.h, pass_mode(dm.K, k, f32), dx, acc);
    else
      hipLaunchKernelGGL((b3_dx<T, false>), dim3(grid), dim3(NT), 0, s, ra, A, B, W1, W3, ls.list,
                         eti, dm.d, dm.h, pass_mode(dm.K, k, f32), dx, acc);
  }
}

hipError_t launch_forward(const FfnPlan& pl, const FfnDims& dm, const void* x, const void* W1,
                          const void* W3, const void* W2, const int32_t* eti,
                          const int32_t* offsets, const int32_t* tim, const float* gates,
                          void* y, void* A, void* B, char* ws, hipStream_t s) {
  if (dm.dtype == 1)
    forward_t<bf16_t>(pl, dm, (const bf16_t*)x, (const bf16_t*)W1, (const bf16_t*)W3,
                      (const bf16_t*)W2, eti, offsets, tim, gates, (bf16_t*)y, (bf16_t*)A,
                      (bf16_t*)B, ws, s);
  else
    forward_t<float>(pl, dm, (const float*)x, (const float*)W1, (const float*)W3,
                     (const float*)W2, eti, offsets, tim, gates, (float*)y, (float*)A, (float*)B,
                     ws, s);
  return hipGetLastError();
}

hipError_t launch_backward(const FfnPlan& pl, const FfnDims& dm, const void* dy, const void* x,
                           const void* W1, const void* W3, const void* W2, const int32_t* eti,
                           const int32_t* offsets, const int32_t* tim, const float* gates,
                           void* A, void* B, void* dx, void* dW1, void* dW3, void* dW2,
                           const int32_t* tei, float* dlogits, char* ws, hipStream_t s) {
  if (dm.dtype == 1)
    backward_t<bf16_t>(pl, dm, (const bf16_t*)dy, (const bf16_t*)x, (const bf16_t*)W1,
                       (const bf16_t*)W3, (const bf16_t*)W2, eti, offsets, tim, gates,
                       (bf16_t*)A, (bf16_t*)B, (bf16_t*)dx, (bf16_t*)dW1, (bf16_t*)dW3,
                       (bf16_t*)dW2, tei, dlogits, ws, s);
  else
    backward_t<float>(pl, dm, (const float*)dy, (const float*)x, (const float*)W1,
                      (const float*)W3, (const float*)W2, eti, offsets, tim, gates, (float*)A,
                      (float*)B, (float*)dx, (float*)dW1, (float*)dW3, (float*)dW2, tei, dlogits,
                      ws, s);
  return hipGetLastError();
}

}  // namespace moe
