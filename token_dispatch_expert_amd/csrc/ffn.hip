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
// GEMM engine (all six GEMMs): 128 x 128 output tile per 256-thread
// workgroup, four wavefronts in a 2 x 2 grid, each wavefront 2 x 2 MFMA
// 32x32 tiles (bf16: v_mfma_f32_32x32x16_bf16; float32: four
// v_mfma_f32_32x32x2f32 per 8-element k group).  One k-tile is 128 bytes of
// k per row (64 bf16 / 32 float32); both operands are staged in LDS with k
// contiguous per row, double buffered, with the next k-tile's global loads
// issued before the current tile's MFMAs.  Operands whose memory layout has
// k contiguous are copied with 16-byte loads; operands with the M/N index
// contiguous (weights in x W, and both sides of the weight-gradient
// products) are loaded as 4 (k) x 16-byte blocks and transposed in
// registers on the way into LDS.
//
// Determinism: every output element has one writer.  The combine into y
// and the input gradient dx run as K ordered slot passes: pass k handles,
// for every token, its route in slot k (ascending expert id), so each token
// row is touched once per pass and the sum over slots is always taken in
// ascending k, in float32.

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int NT = 256;        // threads per workgroup
constexpr int TBM = 128;       // output tile rows
constexpr int TBN = 128;       // output tile columns (logical)
constexpr int ROWB = 128;      // bytes of k per LDS row per k-tile
constexpr int PITCH = ROWB + 16;
constexpr int OPB = 128 * PITCH;         // one operand tile in LDS
constexpr int STAGE = 2 * OPB;           // A + B
constexpr int LDSB = 2 * STAGE;          // double buffered

template <typename T> struct Traits;
template <> struct Traits<bf16_t> {
  static constexpr int ES = 2, VEC = 8, KT = 64;
};
template <> struct Traits<float> {
  static constexpr int ES = 4, VEC = 4, KT = 32;
};

__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  // Workgroups are handed out round-robin over the 8 XCDs; give each XCD a
  // contiguous run of logical tiles so neighbouring tiles share its L2.
  const int64_t per = nblocks >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// ------------------------------------------------------------------ loaders

// Tile of 128 rows with k contiguous in memory.  Thread owns rows
// (tid >> 3) + 32 i (i < 4) and the 16-byte column (tid & 7) of each k-tile.
// Elements k < ksplit come from p0[i] + k, the rest from p1[i] + (k - ksplit).
template <typename T>
struct KLoader {
  const char* p0[4];
  const char* p1[4];
  int ksplit, klen;
  uint4 reg[4];

  __device__ __forceinline__ void fetch(int kt) {
    constexpr int ES = Traits<T>::ES, VEC = Traits<T>::VEC, KT = Traits<T>::KT;
    const int k = kt * KT + (threadIdx.x & 7) * VEC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (p0[i] != nullptr && k < klen) {
        const char* p = k < ksplit ? p0[i] + (int64_t)k * ES : p1[i] + (int64_t)(k - ksplit) * ES;
        v = *reinterpret_cast<const uint4*>(p);
      }
      reg[i] = v;
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int r = threadIdx.x >> 3, c = (threadIdx.x & 7) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(lds + (r + 32 * i) * PITCH + c) = reg[i];
  }
};

// Tile of 128 M/N positions with that index contiguous in memory and k
// indexing rows.  Thread owns k rows kt*KT + kb*4 + i (i < 4) and one
// 16-byte vector of VEC positions starting at logical position nb*VEC.
// Row r(k) = ridx ? ridx[k] : rbase + k; the element sits at col + r * ld.
template <typename T>
struct MNLoader {
  const char* col;
  int64_t ld;            // bytes
  const int32_t* ridx;
  int64_t rbase;
  int klen;
  uint4 reg[4];

  static constexpr int NV = 128 / Traits<T>::VEC;
  __device__ static __forceinline__ int nb() { return threadIdx.x % NV; }
  __device__ static __forceinline__ int kb() { return threadIdx.x / NV; }

  __device__ __forceinline__ void fetch(int kt) {
    constexpr int KT = Traits<T>::KT;
    const int k0 = kt * KT + kb() * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + i;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col != nullptr && k < klen) {
        const int64_t r = ridx != nullptr ? (int64_t)ridx[k] : rbase + k;
        v = *reinterpret_cast<const uint4*>(col + r * ld);
      }
      reg[i] = v;
    }
  }
  __device__ __forceinline__ void store(char* lds) const;
};

template <>
__device__ __forceinline__ void MNLoader<bf16_t>::store(char* lds) const {
  const int n0 = nb() * 8;
  const int kbyte = kb() * 8;
  const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&reg[0]);
  const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&reg[1]);
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&reg[2]);
  const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&reg[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint2 lo, hi;
    lo.x = (q0[w] & 0xffffu) | (q1[w] << 16);
    lo.y = (q2[w] & 0xffffu) | (q3[w] << 16);
    hi.x = (q0[w] >> 16) | (q1[w] & 0xffff0000u);
    hi.y = (q2[w] >> 16) | (q3[w] & 0xffff0000u);
    *reinterpret_cast<uint2*>(lds + (n0 + 2 * w) * PITCH + kbyte) = lo;
    *reinterpret_cast<uint2*>(lds + (n0 + 2 * w + 1) * PITCH + kbyte) = hi;
  }
}

template <>
__device__ __forceinline__ void MNLoader<float>::store(char* lds) const {
  const int n0 = nb() * 4;
  const int kbyte = kb() * 16;
  const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&reg[0]);
  const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&reg[1]);
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&reg[2]);
  const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&reg[3]);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    *reinterpret_cast<uint4*>(lds + (n0 + c) * PITCH + kbyte) = make_uint4(q0[c], q1[c], q2[c], q3[c]);
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
  f32x16_t c[2][2];
};

template <typename T>
__device__ __forceinline__ void mma_ktile(const char* As, const char* Bs, Acc& acc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    uint4 a[2], b[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      a[mt] = *reinterpret_cast<const uint4*>(As + (wm * 64 + mt * 32 + r) * PITCH + kc * 32 + g * 16);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      b[nt] = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + nt * 32 + r) * PITCH + kc * 32 + g * 16);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc.c[mt][nt] = mfma_k8<T>(a[mt], b[nt], acc.c[mt][nt]);
  }
}

// Main loop over nk k-tiles; result in acc (zero when nk == 0).
template <typename T, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, Acc& acc) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc.c[mt][nt][i] = 0.f;
  if (nk <= 0) return;
  la.fetch(0);
  lb.fetch(0);
  la.store(smem);
  lb.store(smem + OPB);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      la.fetch(kt + 1);
      lb.fetch(kt + 1);
    }
    mma_ktile<T>(cur, cur + OPB, acc);
    if (more) {
      la.store(nxt);
      lb.store(nxt + OPB);
    }
    __syncthreads();
  }
}

// Position of accumulator element i of MFMA tile (mt, nt) inside the
// 128 x 128 workgroup tile.
__device__ __forceinline__ int acc_row(int mt, int i) {
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
  return wm * 64 + mt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
}
__device__ __forceinline__ int acc_col(int nt) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
  return wn * 64 + nt * 32 + (lane & 31);
}
// For interleaved dual-B tiles (two matrices, 64 columns each per tile):
// logical column -> (matrix, column within the 64-wide source range).
__device__ __forceinline__ int dual_src(int lc) { return (lc >> 5) & 1; }
__device__ __forceinline__ int dual_col(int lc) { return (lc >> 6) * 32 + (lc & 31); }

template <typename T>
__device__ __forceinline__ float silu_of(float a);
template <>
__device__ __forceinline__ float silu_of<bf16_t>(float a) { return a / (1.0f + __expf(-a)); }
template <>
__device__ __forceinline__ float silu_of<float>(float a) { return a / (1.0f + expf(-a)); }
template <typename T>
__device__ __forceinline__ float sigm_of(float a);
template <>
__device__ __forceinline__ float sigm_of<bf16_t>(float a) { return 1.0f / (1.0f + __expf(-a)); }
template <>
__device__ __forceinline__ float sigm_of<float>(float a) { return 1.0f / (1.0f + expf(-a)); }

// ------------------------------------------------------------------ tiles

// Split each of G segment lists (seg[g*(E+1) + e] .. seg[g*(E+1) + e + 1])
// into row tiles of at most TBM rows.  desc[g][i] = {e, begin, end, 0} or
// {-1, 0, 0, 0} past the last tile.
__global__ __launch_bounds__(256) void tile_table(const int32_t* __restrict__ seg, int E,
                                                  int64_t max_tiles, int4* __restrict__ desc) {
  __shared__ int s_start[257];
  __shared__ int scratch[4];
  const int grp = blockIdx.y;
  const int32_t* off = seg + (int64_t)grp * (E + 1);
  const int tid = threadIdx.x;
  const int n = tid < E ? (off[tid + 1] - off[tid] + TBM - 1) / TBM : 0;
  int tot;
  const int inc = block256_incl_scan(n, scratch, &tot);
  if (tid < E) s_start[tid] = inc - n;
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

// ------------------------------------------------------------------ kernels

struct RouteArgs {            // row tiles over routes or slot-pass lists
  const int4* tiles;
  int64_t ntiles;             // upper bound, rows of the grid
  int nN;                     // column tiles
};

// F1: [A | B] = X W1 [| X W3] with X gathered by expert_token_indices;
// epilogue writes A, B (checkpoint) and G = SiLU(A) [* B].
template <typename T, bool DUAL>
__global__ __launch_bounds__(NT) void f1_gather_glu(RouteArgs ra, const T* __restrict__ x,
                                                    const T* __restrict__ W1,
                                                    const T* __restrict__ W3,
                                                    const int32_t* __restrict__ eti, int d, int h,
                                                    T* __restrict__ A, T* __restrict__ B,
                                                    T* __restrict__ G) {
  __shared__ __attribute__((aligned(16))) char smem[LDSB];
  constexpr int ES = Traits<T>::ES, VEC = Traits<T>::VEC, KT = Traits<T>::KT;
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mtile = lid / ra.nN;
  const int ntile = (int)(lid % ra.nN);
  if (mtile >= ra.ntiles) return;
  const int4 ds = ra.tiles[mtile];
  if (ds.x < 0) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * (DUAL ? 64 : 128);

  KLoader<T> la;
  {
    const int r = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = rb + r + 32 * i;
      la.p0[i] = p < re ? reinterpret_cast<const char*>(x + (int64_t)eti[p] * d) : nullptr;
      la.p1[i] = la.p0[i];
    }
    la.ksplit = d;
    la.klen = d;
  }
  MNLoader<T> lb;
  {
    const int lc = MNLoader<T>::nb() * VEC;
    const int src = DUAL ? dual_src(lc) : 0;
    const int sc = n0 + (DUAL ? dual_col(lc) : lc);
    const T* W = (src == 0 ? W1 : W3) + (int64_t)e * d * h;
    lb.col = sc < h ? reinterpret_cast<const char*>(W + sc) : nullptr;
    lb.ld = (int64_t)h * ES;
    lb.ridx = nullptr;
    lb.rbase = 0;
    lb.klen = d;
  }
  Acc acc;
  gemm_mainloop<T>(la, lb, (d + KT - 1) / KT, smem, acc);

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = rb + acc_row(mt, i);
      if (p >= re) continue;
      if (DUAL) {
        const int c = n0 + dual_col(acc_col(0));
        if (c < h) {
          const float a = acc.c[mt][0][i], b = acc.c[mt][1][i];
          const int64_t o = (int64_t)p * h + c;
          Elem<T>::store(A + o, a);
          Elem<T>::store(B + o, b);
          Elem<T>::store(G + o, silu_of<T>(a) * b);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int c = n0 + acc_col(nt);
          if (c < h) {
            const float a = acc.c[mt][nt][i];
            const int64_t o = (int64_t)p * h + c;
            Elem<T>::store(A + o, a);
            Elem<T>::store(G + o, silu_of<T>(a));
          }
        }
      }
    }
  }
}

// Accumulate one slot pass into the (L, d) output.
//   mode 0: only pass (K == 1): out = v
//   mode 1: first pass:  acc = v
//   mode 2: middle pass: acc += v
//   mode 3: last pass:   out = acc + v
// For float32 outputs `acc` is the output itself (modes 1/2 only).
template <typename T>
__device__ __forceinline__ void combine_store(T* out, float* acc, int64_t o, float v, int mode) {
  if (mode == 0) Elem<T>::store(out + o, v);
  else if (mode == 1) acc[o] = v;
  else if (mode == 2) acc[o] += v;
  else Elem<T>::store(out + o, acc[o] + v);
}

// F2 (slot pass k): O = G W2_e for the pass's rows, y[t] (+)= gate * O.
template <typename T>
__global__ __launch_bounds__(NT) void f2_down_combine(RouteArgs ra, const T* __restrict__ Gb,
                                                      const T* __restrict__ W2,
                                                      const int32_t* __restrict__ list,
                                                      const int32_t* __restrict__ eti,
                                                      const float* __restrict__ gates, int K,
                                                      int k, int d, int h, int mode,
                                                      T* __restrict__ y, float* __restrict__ yacc) {
  __shared__ __attribute__((aligned(16))) char smem[LDSB];
  constexpr int ES = Traits<T>::ES, VEC = Traits<T>::VEC, KT = Traits<T>::KT;
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mtile = lid / ra.nN;
  const int ntile = (int)(lid % ra.nN);
  if (mtile >= ra.ntiles) return;
  const int4 ds = ra.tiles[mtile];
  if (ds.x < 0) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * 128;

  KLoader<T> la;
  {
    const int r = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int li = rb + r + 32 * i;
      la.p0[i] = li < re ? reinterpret_cast<const char*>(Gb + (int64_t)list[li] * h) : nullptr;
      la.p1[i] = la.p0[i];
    }
    la.ksplit = h;
    la.klen = h;
  }
  MNLoader<T> lb;
  {
    const int sc = n0 + MNLoader<T>::nb() * VEC;
    lb.col = sc < d ? reinterpret_cast<const char*>(W2 + (int64_t)e * h * d + sc) : nullptr;
    lb.ld = (int64_t)d * ES;
    lb.ridx = nullptr;
    lb.rbase = 0;
    lb.klen = h;
  }
  Acc acc;
  gemm_mainloop<T>(la, lb, (h + KT - 1) / KT, smem, acc);

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int li = rb + acc_row(mt, i);
      if (li >= re) continue;
      const int64_t t = eti[list[li]];
      const float g = gates[t * K + k];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int c = n0 + acc_col(nt);
        if (c < d) combine_store<T>(y, yacc, t * d + c, g * acc.c[mt][nt][i], mode);
      }
    }
  }
}

// B1: dG = gate * (dy[t] W2_e^T) per route; epilogue recomputes SiLU from
// the checkpoint and writes dA, dB over A, B and Gs = gate * G.
template <typename T, bool DUAL>
__global__ __launch_bounds__(NT) void b1_dgrad_glu(RouteArgs ra, const T* __restrict__ dy,
                                                   const T* __restrict__ W2,
                                                   const int32_t* __restrict__ eti,
                                                   const float* __restrict__ gate_p, int d, int h,
                                                   T* __restrict__ A, T* __restrict__ B,
                                                   T* __restrict__ Gs) {
  __shared__ __attribute__((aligned(16))) char smem[LDSB];
  constexpr int KT = Traits<T>::KT;
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mtile = lid / ra.nN;
  const int ntile = (int)(lid % ra.nN);
  if (mtile >= ra.ntiles) return;
  const int4 ds = ra.tiles[mtile];
  if (ds.x < 0) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * 128;

  KLoader<T> la;
  KLoader<T> lb;
  {
    const int r = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = rb + r + 32 * i;
      la.p0[i] = p < re ? reinterpret_cast<const char*>(dy + (int64_t)eti[p] * d) : nullptr;
      la.p1[i] = la.p0[i];
      const int n = n0 + r + 32 * i;
      lb.p0[i] = n < h ? reinterpret_cast<const char*>(W2 + ((int64_t)e * h + n) * d) : nullptr;
      lb.p1[i] = lb.p0[i];
    }
    la.ksplit = la.klen = d;
    lb.ksplit = lb.klen = d;
  }
  Acc acc;
  gemm_mainloop<T>(la, lb, (d + KT - 1) / KT, smem, acc);

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = rb + acc_row(mt, i);
      if (p >= re) continue;
      const float gp = gate_p[p];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int c = n0 + acc_col(nt);
        if (c >= h) continue;
        const int64_t o = (int64_t)p * h + c;
        const float dg = gp * acc.c[mt][nt][i];
        const float a = Elem<T>::load(A + o);
        const float s = sigm_of<T>(a);
        const float sl = a * s;
        const float ds_ = s * (1.0f + a * (1.0f - s));
        if (DUAL) {
          const float b = Elem<T>::load(B + o);
          Elem<T>::store(A + o, dg * b * ds_);
          Elem<T>::store(B + o, dg * sl);
          Elem<T>::store(Gs + o, gp * sl * b);
        } else {
          Elem<T>::store(A + o, dg * ds_);
          Elem<T>::store(Gs + o, gp * sl);
        }
      }
    }
  }
}

struct WeightArgs {           // weight-gradient tiles: E x nM x nN
  int E, nM, nN;
};

// B0: dW2_e = Gs_e^T dy_e (reduction over the expert's routes, ascending).
template <typename T>
__global__ __launch_bounds__(NT) void b0_dw2(WeightArgs wa, const T* __restrict__ Gs,
                                             const T* __restrict__ dy,
                                             const int32_t* __restrict__ eti,
                                             const int32_t* __restrict__ offsets, int d, int h,
                                             T* __restrict__ dW2) {
  __shared__ __attribute__((aligned(16))) char smem[LDSB];
  constexpr int ES = Traits<T>::ES, VEC = Traits<T>::VEC, KT = Traits<T>::KT;
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_e = (int64_t)wa.nM * wa.nN;
  if (lid >= (int64_t)wa.E * per_e) return;
  const int e = (int)(lid / per_e);
  const int rem = (int)(lid % per_e);
  const int m0 = (rem / wa.nN) * 128, n0 = (rem % wa.nN) * 128;
  const int o0 = offsets[e], n_e = offsets[e + 1] - o0;

  MNLoader<T> la;
  {
    const int sc = m0 + MNLoader<T>::nb() * VEC;
    la.col = sc < h ? reinterpret_cast<const char*>(Gs + sc) : nullptr;
    la.ld = (int64_t)h * ES;
    la.ridx = nullptr;
    la.rbase = o0;
    la.klen = n_e;
  }
  MNLoader<T> lb;
  {
    const int sc = n0 + MNLoader<T>::nb() * VEC;
    lb.col = sc < d ? reinterpret_cast<const char*>(dy + sc) : nullptr;
    lb.ld = (int64_t)d * ES;
    lb.ridx = eti + o0;
    lb.rbase = 0;
    lb.klen = n_e;
  }
  Acc acc;
  gemm_mainloop<T>(la, lb, (n_e + KT - 1) / KT, smem, acc);

  T* out = dW2 + (int64_t)e * h * d;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + acc_row(mt, i);
      if (m >= h) continue;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int c = n0 + acc_col(nt);
        if (c < d) Elem<T>::store(out + (int64_t)m * d + c, acc.c[mt][nt][i]);
      }
    }
}

// B2: dW1_e = X_e^T dA_e [, dW3_e = X_e^T dB_e], X gathered by
// expert_token_indices; both products share the X tile (interleaved columns).
template <typename T, bool DUAL>
__global__ __launch_bounds__(NT) void b2_dw13(WeightArgs wa, const T* __restrict__ x,
                                              const T* __restrict__ dA,
                                              const T* __restrict__ dB,
                                              const int32_t* __restrict__ eti,
                                              const int32_t* __restrict__ offsets, int d, int h,
                                              T* __restrict__ dW1, T* __restrict__ dW3) {
  __shared__ __attribute__((aligned(16))) char smem[LDSB];
  constexpr int ES = Traits<T>::ES, VEC = Traits<T>::VEC, KT = Traits<T>::KT;
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_e = (int64_t)wa.nM * wa.nN;
  if (lid >= (int64_t)wa.E * per_e) return;
  const int e = (int)(lid / per_e);
  const int rem = (int)(lid % per_e);
  const int m0 = (rem / wa.nN) * 128, n0 = (rem % wa.nN) * (DUAL ? 64 : 128);
  const int o0 = offsets[e], n_e = offsets[e + 1] - o0;

  MNLoader<T> la;
  {
    const int sc = m0 + MNLoader<T>::nb() * VEC;
    la.col = sc < d ? reinterpret_cast<const char*>(x + sc) : nullptr;
    la.ld = (int64_t)d * ES;
    la.ridx = eti + o0;
    la.rbase = 0;
    la.klen = n_e;
  }
  MNLoader<T> lb;
  {
    const int lc = MNLoader<T>::nb() * VEC;
    const int src = DUAL ? dual_src(lc) : 0;
    const int sc = n0 + (DUAL ? dual_col(lc) : lc);
    const T* S = src == 0 ? dA : dB;
    lb.col = sc < h ? reinterpret_cast<const char*>(S + sc) : nullptr;
    lb.ld = (int64_t)h * ES;
    lb.ridx = nullptr;
    lb.rbase = o0;
    lb.klen = n_e;
  }
  Acc acc;
  gemm_mainloop<T>(la, lb, (n_e + KT - 1) / KT, smem, acc);

  T* o1 = dW1 + (int64_t)e * d * h;
  T* o3 = DUAL ? dW3 + (int64_t)e * d * h : nullptr;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
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
        for (int nt = 0; nt < 2; ++nt) {
          const int c = n0 + acc_col(nt);
          if (c < h) Elem<T>::store(o1 + (int64_t)m * h + c, acc.c[mt][nt][i]);
        }
      }
    }
}

// B3 (slot pass k): dX = [dA | dB] [W1_e | W3_e]^T for the pass's rows,
// dx[t] (+)= dX.  One GEMM over the concatenated 2h.
template <typename T, bool DUAL>
__global__ __launch_bounds__(NT) void b3_dx(RouteArgs ra, const T* __restrict__ dA,
                                            const T* __restrict__ dB, const T* __restrict__ W1,
                                            const T* __restrict__ W3,
                                            const int32_t* __restrict__ list,
                                            const int32_t* __restrict__ eti, int d, int h,
                                            int mode, T* __restrict__ dx,
                                            float* __restrict__ dxacc) {
  __shared__ __attribute__((aligned(16))) char smem[LDSB];
  constexpr int KT = Traits<T>::KT;
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mtile = lid / ra.nN;
  const int ntile = (int)(lid % ra.nN);
  if (mtile >= ra.ntiles) return;
  const int4 ds = ra.tiles[mtile];
  if (ds.x < 0) return;
  const int e = ds.x, rb = ds.y, re = ds.z;
  const int n0 = ntile * 128;
  const int klen = DUAL ? 2 * h : h;

  KLoader<T> la;
  KLoader<T> lb;
  {
    const int r = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int li = rb + r + 32 * i;
      const int64_t p = li < re ? (int64_t)list[li] : -1;
      la.p0[i] = p >= 0 ? reinterpret_cast<const char*>(dA + p * h) : nullptr;
      la.p1[i] = (p >= 0 && DUAL) ? reinterpret_cast<const char*>(dB + p * h) : la.p0[i];
      const int n = n0 + r + 32 * i;
      lb.p0[i] = n < d ? reinterpret_cast<const char*>(W1 + ((int64_t)e * d + n) * h) : nullptr;
      lb.p1[i] = (n < d && DUAL) ? reinterpret_cast<const char*>(W3 + ((int64_t)e * d + n) * h) : lb.p0[i];
    }
    la.ksplit = lb.ksplit = h;
    la.klen = lb.klen = klen;
  }
  Acc acc;
  gemm_mainloop<T>(la, lb, (klen + KT - 1) / KT, smem, acc);

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int li = rb + acc_row(mt, i);
      if (li >= re) continue;
      const int64_t t = eti[list[li]];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int c = n0 + acc_col(nt);
        if (c < d) combine_store<T>(dx, dxacc, t * d + c, acc.c[mt][nt][i], mode);
      }
    }
  }
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
  size_t o = 0;
  p.off_g = o;      o = align_up(o + (size_t)p.R * dm.h * es, 256);
  p.off_acc = o;    o = align_up(o + (need_acc ? (size_t)dm.L * dm.d * 4 : 0), 256);
  p.off_slot = o;   o = align_up(o + (size_t)p.R + 16, 256);
  p.off_list = o;   o = align_up(o + (size_t)p.R * 4, 256);
  p.off_cnt = o;    o = align_up(o + (size_t)dm.K * p.list_chunks * 4, 256);
  p.off_base = o;   o = align_up(o + (size_t)dm.K * p.list_chunks * 4, 256);
  p.off_peoff = o;  o = align_up(o + (size_t)dm.K * (dm.E + 1) * 4, 256);
  p.off_gatep = o;  o = align_up(o + (backward ? (size_t)p.R * 4 : 0), 256);
  p.off_tiles_route = o; o = align_up(o + (size_t)p.route_tiles * 16, 256);
  p.off_tiles_pass = o;  o = align_up(o + (size_t)dm.K * p.pass_tiles * 16, 256);
  p.bytes = o;
  return p;
}

struct Lists {
  int32_t* list;
  int32_t* pe_off;
  int4* tiles_route;
  int4* tiles_pass;
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
  const int C = (int)pl.list_chunks;
  {
    LaunchTimer lt("route_tiles", s);
    hipLaunchKernelGGL(tile_table, dim3((unsigned)cdiv(pl.route_tiles, 256), 1), dim3(256), 0, s,
                       offsets, dm.E, pl.route_tiles, ls.tiles_route);
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
                       s, ls.pe_off, dm.E, pl.pass_tiles, ls.tiles_pass);
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
static void forward_t(const FfnPlan& pl, const FfnDims& dm, const T* x, const T* W1, const T* W3,
                      const T* W2, const int32_t* eti, const int32_t* offsets, const int32_t* tim,
                      const float* gates, T* y, T* A, T* B, char* ws, hipStream_t s) {
  const bool f32 = sizeof(T) == 4;
  const bool dual = dm.act == 1;
  Lists ls = build_lists(pl, dm, offsets, tim, gates, nullptr, ws, s);
  T* G = reinterpret_cast<T*>(ws + pl.off_g);
  float* acc = f32 ? reinterpret_cast<float*>(y) : reinterpret_cast<float*>(ws + pl.off_acc);
  {
    LaunchTimer lt("ffn_f1_gather_glu", s);
    RouteArgs ra{ls.tiles_route, pl.route_tiles, (int)cdiv(dm.h, dual ? 64 : 128)};
    const unsigned grid = (unsigned)round8(ra.ntiles * ra.nN);
    if (dual)
      hipLaunchKernelGGL((f1_gather_glu<T, true>), dim3(grid), dim3(NT), 0, s, ra, x, W1, W3, eti,
                         dm.d, dm.h, A, B, G);
    else
      hipLaunchKernelGGL((f1_gather_glu<T, false>), dim3(grid), dim3(NT), 0, s, ra, x, W1, W3,
                         eti, dm.d, dm.h, A, B, G);
  }
  for (int k = 0; k < dm.K; ++k) {
    LaunchTimer lt("ffn_f2_down_combine", s);
    RouteArgs ra{ls.tiles_pass + (int64_t)k * pl.pass_tiles, pl.pass_tiles, (int)cdiv(dm.d, 128)};
    const unsigned grid = (unsigned)round8(ra.ntiles * ra.nN);
    hipLaunchKernelGGL((f2_down_combine<T>), dim3(grid), dim3(NT), 0, s, ra, G, W2, ls.list, eti,
                       gates, dm.K, k, dm.d, dm.h, pass_mode(dm.K, k, f32), y, acc);
  }
}

template <typename T>
static void backward_t(const FfnPlan& pl, const FfnDims& dm, const T* dy, const T* x, const T* W1,
                       const T* W3, const T* W2, const int32_t* eti, const int32_t* offsets,
                       const int32_t* tim, const float* gates, T* A, T* B, T* dx, T* dW1, T* dW3,
                       T* dW2, char* ws, hipStream_t s) {
  const bool f32 = sizeof(T) == 4;
  const bool dual = dm.act == 1;
  float* gate_p = reinterpret_cast<float*>(ws + pl.off_gatep);
  Lists ls = build_lists(pl, dm, offsets, tim, gates, gate_p, ws, s);
  T* Gs = reinterpret_cast<T*>(ws + pl.off_g);
  float* acc = f32 ? reinterpret_cast<float*>(dx) : reinterpret_cast<float*>(ws + pl.off_acc);
  {
    LaunchTimer lt("ffn_b1_dgrad_glu", s);
    RouteArgs ra{ls.tiles_route, pl.route_tiles, (int)cdiv(dm.h, 128)};
    const unsigned grid = (unsigned)round8(ra.ntiles * ra.nN);
    if (dual)
      hipLaunchKernelGGL((b1_dgrad_glu<T, true>), dim3(grid), dim3(NT), 0, s, ra, dy, W2, eti,
                         gate_p, dm.d, dm.h, A, B, Gs);
    else
      hipLaunchKernelGGL((b1_dgrad_glu<T, false>), dim3(grid), dim3(NT), 0, s, ra, dy, W2, eti,
                         gate_p, dm.d, dm.h, A, B, Gs);
  }
  {
    LaunchTimer lt("ffn_b0_dw2", s);
    WeightArgs wa{dm.E, (int)cdiv(dm.h, 128), (int)cdiv(dm.d, 128)};
    const int64_t n = (int64_t)dm.E * wa.nM * wa.nN;
    hipLaunchKernelGGL((b0_dw2<T>), dim3((unsigned)round8(n)), dim3(NT), 0, s, wa, Gs, dy, eti,
                       offsets, dm.d, dm.h, dW2);
  }
  {
    LaunchTimer lt("ffn_b2_dw13", s);
    WeightArgs wa{dm.E, (int)cdiv(dm.d, 128), (int)cdiv(dm.h, dual ? 64 : 128)};
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
    RouteArgs ra{ls.tiles_pass + (int64_t)k * pl.pass_tiles, pl.pass_tiles, (int)cdiv(dm.d, 128)};
    const unsigned grid = (unsigned)round8(ra.ntiles * ra.nN);
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
                           char* ws, hipStream_t s) {
  if (dm.dtype == 1)
    backward_t<bf16_t>(pl, dm, (const bf16_t*)dy, (const bf16_t*)x, (const bf16_t*)W1,
                       (const bf16_t*)W3, (const bf16_t*)W2, eti, offsets, tim, gates,
                       (bf16_t*)A, (bf16_t*)B, (bf16_t*)dx, (bf16_t*)dW1, (bf16_t*)dW3,
                       (bf16_t*)dW2, ws, s);
  else
    backward_t<float>(pl, dm, (const float*)dy, (const float*)x, (const float*)W1,
                      (const float*)W3, (const float*)W2, eti, offsets, tim, gates, (float*)A,
                      (float*)B, (float*)dx, (float*)dW1, (float*)dW3, (float*)dW2, ws, s);
  return hipGetLastError();
}

}  // namespace moe
