// Atomic-free construction of the routing index structures on gfx950.
//
// The three steps follow the MoEBlaze wiki note, "Core method" >
// "atomic-free three-step dispatch construction":
//   1. a dense token-expert map, each (expert, token) entry written once;
//   2. per-expert length counts by reduction, then a prefix sum for the
//      expert offsets;
//   3. a scan inside each tile of the map gives every selected entry its
//      final place in the per-expert token list, then a parallel write.
//
// MI355X layout.  The map is stored expert-major, [E][Lpad] bytes, holding
// slot+1 for a selected entry and 0 otherwise (the slot is needed to fill
// token_index_map).  Step 1 routes one tile of T tokens per workgroup and
// transposes its part of the map through LDS so that every map row segment
// leaves as full 16-byte stores; as a by-product it counts each expert's
// entries in the tile, so step 2 only has to scan E x C tile counts (one
// workgroup per expert column) instead of re-reading the map.  Step 3 reads
// each row segment once with 16-byte loads, one wavefront per expert row.
// No kernel uses atomics; every output element has exactly one writer.

#include "moe_device.h"
#include "moe_internal.h"

#include <limits.h>

namespace moe {

// Step 1: top-K routing, gates, map tile, per-tile expert counts.
// G lanes cooperate on one token; lane j of the group owns experts
// 4j .. 4j+3.  The K winners are found by K rounds of a group arg-max (ties
// to the lower expert id); the softmax and the ascending-expert slot order
// come from group reductions and a group prefix count.  NaN logits (outside
// the contract) rank as -inf in the arg-max, so a token with fewer than K
// other logits still gets K distinct experts, filled from the lowest ids.
template <int G>
__device__ __forceinline__ void route_token(const float (&v)[4], int lg, int E, int K, int64_t t,
                                            int tl, int T, int32_t* __restrict__ tei,
                                            float* __restrict__ gates, uint8_t* smap) {
  int ev[4];
  // selection key: a NaN logit (outside the contract) ranks as -inf, so that
  // every round still finds an expert and each token gets K distinct ones
  float key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ev[j] = lg * 4 + j;
    key[j] = v[j] == v[j] ? v[j] : -INFINITY;
  }
  unsigned sel = 0;
  float vmax = 0.f;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = INT_MAX;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool cand = !((sel >> j) & 1u) && ev[j] < E;
      if (cand && (key[j] > bv || (key[j] == bv && ev[j] < be))) {
        bv = key[j];
        be = ev[j];
      }
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, G);
      const int oe = __shfl_xor(be, o, G);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (k == 0) vmax = bv;
    if ((be >> 2) == lg) sel |= 1u << (be & 3);
  }
  float ssum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if ((sel >> j) & 1u) ssum += expf(v[j] - vmax);
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) ssum += __shfl_xor(ssum, o, G);
  const int c = __popc(sel);
  int inc = c;
#pragma unroll
  for (int o = 1; o < G; o <<= 1) {
    const int u = __shfl_up(inc, o, G);
    if (lg >= o) inc += u;
  }
  int slot = inc - c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if ((sel >> j) & 1u) {
      tei[t * K + slot] = ev[j];
      gates[t * K + slot] = expf(v[j] - vmax) / ssum;
      smap[ev[j] * T + tl] = (uint8_t)(slot + 1);
      ++slot;
    }
  }
}

// The logits of one token for lane lg of its group (-inf where absent).
// Loads never branch: a missing token or expert reads a valid address and
// is replaced by -inf.
template <bool VEC4>
__device__ __forceinline__ void load_logits(const float* __restrict__ logits, int64_t t, bool ok,
                                            int E, int lg, float (&v)[4]) {
  const float* row = logits + (ok ? t : 0) * E;
  if (VEC4) {
    const bool in = ok && lg * 4 < E;
    const float4 q = *reinterpret_cast<const float4*>(row + (in ? lg * 4 : 0));
    v[0] = in ? q.x : -INFINITY;
    v[1] = in ? q.y : -INFINITY;
    v[2] = in ? q.z : -INFINITY;
    v[3] = in ? q.w : -INFINITY;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lg * 4 + j;
      const bool in = ok && e < E;
      const float q = row[in ? e : 0];
      v[j] = in ? q : -INFINITY;
    }
  }
}

// One workgroup per tile of T tokens.  The tile's logits are read U token
// groups at a time, all loads issued before any routing, so that each lane
// keeps U 16-byte loads in flight.  The map tile [E][T] is built in LDS
// (dynamic, E*T <= 64 KB) and leaves as 16-byte row stores.
template <int G, bool VEC4>
__global__ __launch_bounds__(256) void k1_route_map(const float* __restrict__ logits, int64_t L,
                                                    int E, int K, int T, int C, int64_t Lpad,
                                                    int32_t* __restrict__ tei,
                                                    float* __restrict__ gates,
                                                    uint8_t* __restrict__ map,
                                                    int32_t* __restrict__ tilecnt) {
  extern __shared__ uint4 smap_v[];
  uint8_t* smap = reinterpret_cast<uint8_t*>(smap_v);
  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * T;
  const int nvec = (E * T) >> 4;
  for (int i = threadIdx.x; i < nvec; i += 256) smap_v[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int lg = threadIdx.x & (G - 1);
  constexpr int NG = 256 / G;
  constexpr int U = 8;
  for (int b0 = threadIdx.x / G; b0 < T; b0 += NG * U) {
    float v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tl = b0 + u * NG;
      const int64_t t = t0 + tl;
      load_logits<VEC4>(logits, t, tl < T && t < L, E, lg, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tl = b0 + u * NG;
      const int64_t t = t0 + tl;
      if (tl < T && t < L) route_token<G>(v[u], lg, E, K, t, tl, T, tei, gates, smap);
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = T >> 4;
  for (int e = wave; e < E; e += 4) {
    int cnt = 0;
    for (int i = lane; i < nv; i += 64) {
      const uint4 q = smap_v[(e * T >> 4) + i];
      *reinterpret_cast<uint4*>(map + (int64_t)e * Lpad + t0 + i * 16) = q;
      cnt += nonzero_bytes(q.x) + nonzero_bytes(q.y) + nonzero_bytes(q.z) + nonzero_bytes(q.w);
    }
    cnt = wave_sum(cnt);
    if (lane == 0) tilecnt[(int64_t)e * C + tile] = cnt;
  }
}

// Step 1 for E <= 64: one thread per token with the token's logits in
// registers (EV = E rounded up to a multiple of 4).  Top-K is K register
// passes of an arg-max with ties to the lower id; no cross-lane traffic.
template <int EV>
__global__ __launch_bounds__(256) void k1_route_map_rows(const float* __restrict__ logits,
                                                         int64_t L, int E, int K, int T, int C,
                                                         int64_t Lpad, int32_t* __restrict__ tei,
                                                         float* __restrict__ gates,
                                                         uint8_t* __restrict__ map,
                                                         int32_t* __restrict__ tilecnt) {
  extern __shared__ uint4 smap_v[];
  uint8_t* smap = reinterpret_cast<uint8_t*>(smap_v);
  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * T;
  const int nvec = (E * T) >> 4;
  for (int i = threadIdx.x; i < nvec; i += 256) smap_v[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  for (int tl = threadIdx.x; tl < T; tl += 256) {
    const int64_t t = t0 + tl;
    if (t >= L) break;
    float v[EV];
    const float4* row = reinterpret_cast<const float4*>(logits + t * E);
#pragma unroll
    for (int j = 0; j < EV / 4; ++j) {
      // E is a multiple of 4 here; vectors past the row are not read.
      float4 q = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (4 * j < E) q = row[j];
      v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
    }
    uint64_t sel = 0;
    float vmax = 0.f;
    for (int k = 0; k < K; ++k) {
      float bv = -INFINITY;
      int be = -1;
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        const bool cand = e < E && !((sel >> e) & 1ull);
        if (cand && (be < 0 || v[e] > bv)) {
          bv = v[e];
          be = e;
        }
      }
      if (k == 0) vmax = bv;
      sel |= 1ull << be;
    }
    float ssum = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e)
      if ((sel >> e) & 1ull) ssum += expf(v[e] - vmax);
    int slot = 0;
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      if ((sel >> e) & 1ull) {
        tei[t * K + slot] = e;
        gates[t * K + slot] = expf(v[e] - vmax) / ssum;
        smap[e * T + tl] = (uint8_t)(slot + 1);
        ++slot;
      }
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = T >> 4;
  for (int e = wave; e < E; e += 4) {
    int cnt = 0;
    for (int i = lane; i < nv; i += 64) {
      const uint4 q = smap_v[(e * T >> 4) + i];
      *reinterpret_cast<uint4*>(map + (int64_t)e * Lpad + t0 + i * 16) = q;
      cnt += nonzero_bytes(q.x) + nonzero_bytes(q.y) + nonzero_bytes(q.z) + nonzero_bytes(q.w);
    }
    cnt = wave_sum(cnt);
    if (lane == 0) tilecnt[(int64_t)e * C + tile] = cnt;
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int lowest_bit(uint64_t m) { return __builtin_ctzll(m); }

// Step 1, streaming form (E <= EB <= 64, K <= KM <= 8).  One wavefront per
// workgroup routes one 64-token part, one token per lane (small workgroups
// keep many parts in flight per CU).  The part's logit rows are one
// contiguous run of 256 E bytes, copied straight into LDS with 1 KB
// global_load_lds transfers (from the 16-byte boundary at or below its start,
// so any 4-byte aligned logits work).  Each lane reads its own row back in
// 4-element chunks, starting at a lane-dependent chunk so that the lanes of
// one LDS cycle hit different banks.  VEC: E % 4 == 0 and 16-byte aligned
// rows, read as float4.
//
// Selection is exact top-K with ties to the lower expert id, done in two
// passes over the row instead of K arg-max passes:
//   pass 1 keeps the KM largest values as a descending register list; a new
//          value x enters as b[0] = max(b[0], x), b[i] = med3(b[i-1], b[i], x)
//          (one instruction per slot, no index bookkeeping);
//   pass 2 marks every expert whose logit is >= b[K-1] in a 64-bit mask.
// The mask has at least K bits; extra bits can only be ties with b[K-1], and
// dropping those of the highest ids leaves the lower-id choice.  Slots are the
// mask bits in ascending id order.  NaN logits (outside the contract) cannot
// produce an invalid id: the mask is trimmed or filled to exactly K bits.
//
// Outputs besides tei and gates (the token-expert map of the method, in bit
// form): each token's expert mask; for each part and expert e the column
// col[part][e] (bit j set = token j of the part chose e); and the part's
// per-expert counts cnt[e][part].
// Transposes a wavefront's expert masks one expert at a time (for masks of
// at most 32 experts): for e in [E0, EB), lane e of (hi:lo) receives the
// ballot of bit e of m (bit j = lane j has bit e set).
template <int E0, int EB>
struct BallotColumns {
  static __device__ __forceinline__ void run(uint64_t m, uint32_t& lo, uint32_t& hi) {
    const uint64_t bal = __ballot((m >> E0) & 1);
    // the ballot was just written by a VALU compare: two wait states before
    // it is read (the hazard checker does not look inside inline asm)
    asm("s_nop 1\n\tv_writelane_b32 %0, %2, %4\n\tv_writelane_b32 %1, %3, %4"
        : "=v"(lo), "=v"(hi)
        : "s"((uint32_t)bal), "s"((uint32_t)(bal >> 32)), "i"(E0), "0"(lo), "1"(hi));
    BallotColumns<E0 + 1, EB>::run(m, lo, hi);
  }
};
template <int EB>
struct BallotColumns<EB, EB> {
  static __device__ __forceinline__ void run(uint64_t, uint32_t&, uint32_t&) {}
};

// 64 x 64 bit transpose across the wavefront: lane j holds row j (bit e =
// token j chose expert e); on return lane e holds column e (bit j = token j
// chose e).  Six exchange stages of the block transpose: at stage j the lane
// pairs (k, k + j), k with lane bit j clear, swap the upper-right and
// lower-left j x j blocks of their two rows.
__device__ __forceinline__ uint64_t wave_transpose64(uint64_t x, int lane) {
  constexpr uint64_t kMask[6] = {0x00000000FFFFFFFFull, 0x0000FFFF0000FFFFull,
                                 0x00FF00FF00FF00FFull, 0x0F0F0F0F0F0F0F0Full,
                                 0x3333333333333333ull, 0x5555555555555555ull};
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int j = 32 >> s;
    const uint32_t plo = (uint32_t)__shfl_xor((int)(uint32_t)x, j, 64);
    const uint32_t phi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), j, 64);
    const uint64_t y = ((uint64_t)phi << 32) | plo;
    const bool top = (lane & j) == 0;
    const uint64_t a = top ? x : y, b = top ? y : x;  // rows k and k + j
    const uint64_t t = ((a >> j) ^ b) & kMask[s];
    x ^= top ? (t << j) : t;
  }
  return x;
}

struct RouteSrc {
  const char* abase;  // logits rounded down to 16 bytes
  int64_t mis;        // logits - abase
  int64_t end16;      // readable bytes from abase (rounded up to 16)
};

// Issue the copy of part `part` into `dst`; returns the offset of its first
// row inside `dst`.  NT: copy with the non-temporal hint (the logits are read
// once; measured faster for 64-expert rows, slower for 16).
template <bool NT>
__device__ __forceinline__ int copy_part(const RouteSrc& src, int64_t part, int rowb, int64_t L,
                                         char* dst, int lane) {
  const int64_t first = src.mis + part * 64 * rowb;
  const int64_t first16 = first & ~(int64_t)15;
  const int delta = (int)(first - first16);
  const int nq = part * 64 < L ? (int)((delta + 64 * rowb + 1023) >> 10) : 0;
  for (int q = 0; q < nq; ++q) {
    const int64_t off = first16 + q * 1024 + lane * 16;
    const char* g = src.abase + (off + 16 <= src.end16 ? off : 0);
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + q * 1024), 16, 0, NT ? 2 : 0);
  }
  return delta;
}

template <int EB, int KM, bool VEC>
__device__ __forceinline__ uint64_t route_row(const float* row, int E, int K, int lane, bool live,
                                              int64_t t, int32_t* __restrict__ tei,
                                              float* __restrict__ gates) {
  const int nc = (E + 3) >> 2;
  const int rot = lane % nc;
  auto chunk = [&](int c, float (&v)[4]) {
    if (VEC) {
      const float4 q = reinterpret_cast<const float4*>(row)[c];
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = (4 * c + u < E) ? row[4 * c + u] : -INFINITY;
    }
  };
  float b[KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) b[i] = -INFINITY;
  for (int j = 0, c = rot; j < nc; ++j, c = (c + 1 == nc) ? 0 : c + 1) {
    float v[4];
    chunk(c, v);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int i = KM - 1; i > 0; --i) b[i] = __builtin_amdgcn_fmed3f(b[i - 1], b[i], v[u]);
      b[0] = fmaxf(b[0], v[u]);
    }
  }
  float thr = b[0];
#pragma unroll
  for (int i = 1; i < KM; ++i) thr = (i == K - 1) ? b[i] : thr;

  uint64_t m = 0;
  for (int j = 0, c = rot; j < nc; ++j, c = (c + 1 == nc) ? 0 : c + 1) {
    float v[4];
    chunk(c, v);
    const uint32_t m4 = (v[0] >= thr ? 1u : 0u) | (v[1] >= thr ? 2u : 0u) |
                        (v[2] >= thr ? 4u : 0u) | (v[3] >= thr ? 8u : 0u);
    m |= (uint64_t)m4 << (4 * c);
  }
  if (!VEC && E < 64) m &= (1ull << E) - 1;  // padding of the last chunk
  int cnt = __builtin_popcountll(m);
  for (int e = E - 1; e >= 0 && cnt > K; --e) {
    if (((m >> e) & 1) && !(row[e] > thr)) {
      m &= ~(1ull << e);
      --cnt;
    }
  }
  for (int e = 0; e < E && cnt < K; ++e) {
    if (!((m >> e) & 1)) {
      m |= 1ull << e;
      ++cnt;
    }
  }
  if (!live) return 0;

  const float vmax = b[0];
  float ssum = 0.f;
#pragma unroll
  for (int i = 0; i < KM; ++i)
    if (i < K) ssum += expf(b[i] - vmax);
  const float inv = 1.0f / ssum;
  uint64_t mm = m;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k < K) {
      const int e = lowest_bit(mm);
      mm &= mm - 1;
      tei[t * K + k] = e;
      gates[t * K + k] = expf(row[e] - vmax) * inv;
    }
  }
  return m;
}

template <int EB, int KM, bool VEC>
__global__ __launch_bounds__(64) void k1_route_mask(const float* __restrict__ logits, int64_t L,
                                                    int E, int K, int64_t NP,
                                                    int32_t* __restrict__ tei,
                                                    float* __restrict__ gates,
                                                    uint64_t* __restrict__ tmask,
                                                    uint64_t* __restrict__ tcol,
                                                    int32_t* __restrict__ partcnt) {
  constexpr int PART = 64 * 4 * EB + (VEC ? 0 : 1024);  // LDS bytes
  __shared__ __attribute__((aligned(16))) char stage[PART];
  const int lane = threadIdx.x;
  int64_t part;
  {  // contiguous runs of parts per XCD: neighbouring parts' count words meet in one L2
    const int64_t nb = gridDim.x, b = blockIdx.x, q = nb >> 3, r = nb & 7, x = b & 7;
    part = x * q + (x < r ? x : r) + (b >> 3);
  }
  const int rowb = 4 * E;
  RouteSrc src;
  {
    const char* lbase = reinterpret_cast<const char*>(logits);
    src.mis = (int64_t)(reinterpret_cast<uintptr_t>(lbase) & 15);  // 0 when VEC
    src.abase = lbase - src.mis;
    src.end16 = (src.mis + L * rowb + 15) & ~(int64_t)15;
  }
  const int delta = copy_part<(EB >= 64)>(src, part, rowb, L, stage, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const int64_t t = part * 64 + lane;
  const float* row = reinterpret_cast<const float*>(stage + delta + lane * rowb);
  const uint64_t m = route_row<EB, KM, VEC>(row, E, K, lane, t < L, t, tei, gates);
  if (t < L) tmask[t] = m;
  // the part's column of the map for expert e, kept by lane e (bits of
  // experts >= E are clear, so their columns are empty): a bit transpose of
  // the 64 masks for 64-expert rows, one ballot per expert for narrower ones
  uint64_t mycol;
  if constexpr (EB == 64) {
    mycol = wave_transpose64(m, lane);
  } else {
    uint32_t col_lo = 0, col_hi = 0;
    BallotColumns<0, EB>::run(m, col_lo, col_hi);
    mycol = ((uint64_t)col_hi << 32) | col_lo;
  }
  if (lane < E) {
    tcol[part * E + lane] = mycol;
    partcnt[(int64_t)lane * NP + part] = __popcll(mycol);
  }
}

// Step 1, streaming form for exactly 64 experts with 16-byte aligned rows
// and L >= 64: as k1_route_mask, but the part's 16 KB of logits come in
// through registers (sixteen coalesced 16-byte loads per lane, all in flight
// together) and the wavefront writes them into LDS itself, which moves
// 256-byte rows faster than the direct-to-LDS copies.  The last part reads
// rows [L - 64, L) instead of running past the end, so every load is in
// range; token t then sits in stage row t - first_row.
template <int KM>
__global__ __launch_bounds__(64) void k1_route_mask64(const float* __restrict__ logits, int64_t L,
                                                      int E, int K, int64_t NP,
                                                      int32_t* __restrict__ tei,
                                                      float* __restrict__ gates,
                                                      uint64_t* __restrict__ tmask,
                                                      uint64_t* __restrict__ tcol,
                                                      int32_t* __restrict__ partcnt) {
  constexpr int NQ = 16;  // 16-byte loads per lane (E == 64)
  typedef float v4f __attribute__((ext_vector_type(4)));
  __shared__ v4f stage[64 * NQ];
  const int lane = threadIdx.x;
  int64_t part;
  {  // contiguous runs of parts per XCD: neighbouring parts' count words meet in one L2
    const int64_t nb = gridDim.x, b = blockIdx.x, q = nb >> 3, r = nb & 7, x = b & 7;
    part = x * q + (x < r ? x : r) + (b >> 3);
  }
  const int64_t first_row = min(part * 64, L - 64);
  const v4f* pb = reinterpret_cast<const v4f*>(logits) + first_row * NQ;  // uniform
  v4f v[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c) v[c] = __builtin_nontemporal_load(pb + c * 64 + lane);
#pragma unroll
  for (int c = 0; c < NQ; ++c) stage[c * 64 + lane] = v[c];
  __builtin_amdgcn_wave_barrier();
  const int64_t t = part * 64 + lane;
  // rows past L (last part only) route a valid row and store nothing
  const int srow = (int)min<int64_t>(t - first_row, 63);
  // E (64) comes in as an argument: the selection then loops over the row's
  // chunks instead of unrolling all of them into registers
  const float* row = reinterpret_cast<const float*>(stage) + srow * E;
  const uint64_t m = route_row<64, KM, true>(row, E, K, lane, t < L, t, tei, gates);
  if (t < L) tmask[t] = m;
  const uint64_t mycol = wave_transpose64(m, lane);  // m = 0 past L
  tcol[part * E + lane] = mycol;
  partcnt[(int64_t)lane * NP + part] = __popcll(mycol);
}

// Step 3 for the streaming form: one workgroup per 256-token tile, one
// wavefront per 64-token part.  A token's position in expert e's segment is
// the segment start, plus the tokens of e in earlier tiles (scanned counts),
// plus those in earlier parts of this tile, plus the set bits of the part's
// column col[e] below its lane.  Tokens therefore appear in ascending order
// within each segment, and the tile's tokens of one expert occupy one run of
// that segment: the tile collects its entries in LDS ordered by expert and
// writes them out run by run.  Tiles are spread over the XCDs in contiguous
// ranges so that neighbouring runs meet in one L2.
template <int RW, int KMAX>
__global__ __launch_bounds__(256) void k3_scatter_mask(const uint64_t* __restrict__ tmask,
                                                       const uint64_t* __restrict__ tcol,
                                                       int64_t L, int E, int K, int NU,
                                                       const int32_t* __restrict__ unitbase,
                                                       const int32_t* __restrict__ total,
                                                       int32_t* __restrict__ eti,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tim) {
  // entries of one tile (K <= KMAX): the staging arrays are sized for the
  // layer's K bucket, so that smaller K leaves room for more workgroups per CU
  constexpr int MAXE = 256 * KMAX;
  __shared__ int s_off[257];
  __shared__ int scratch[4];
  __shared__ uint64_t s_col[4][64];
  __shared__ int s_ub[4][64];
  __shared__ int s_base[4][64];
  __shared__ int s_run[65];  // start of each expert's run inside the tile
  __shared__ int s_tok[MAXE];
  // expert of each staged entry; its position in expert_token_indices is the
  // entry's index plus s_dl[e] (the tile's run of e lies in one run of e's
  // segment), which saves a 4-byte position per entry: 8 workgroups per CU
  // at K = 6 instead of 6
  __shared__ uint8_t s_ex[MAXE];
  __shared__ int s_dl[64];
  __shared__ int s_tim[MAXE];  // the tile's token_index_map rows, written out contiguously
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int tile;
  {
    const int nb = gridDim.x, b = blockIdx.x, q = nb >> 3, r = nb & 7, x = b & 7;
    tile = x * q + (x < r ? x : r) + (b >> 3);
  }
  const int64_t part = (int64_t)tile * 4 + wave;
  const int64_t t = part * 64 + lane;
  const bool part_live = part * 64 < L;
  const int64_t unit = part / RW;

  // independent loads first
  const int v = tid < E ? total[tid] : 0;
  const uint64_t colv = (lane < E && part_live) ? tcol[part * E + lane] : 0;
  const int ub = (lane < E && part_live && wave % RW == 0) ? unitbase[(int64_t)lane * NU + unit] : 0;
  uint64_t m = t < L ? tmask[t] : 0;

  int tot;
  const int inc = block256_incl_scan(v, scratch, &tot);
  if (tid < E) s_off[tid] = inc - v;
  if (tid == 0) s_off[E] = tot;
  if (lane < E) {
    s_col[wave][lane] = colv;
    s_ub[wave][lane] = ub;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) offsets[tid] = s_off[tid];
    if (tid == 0) offsets[E] = s_off[E];
  }
  if (wave == 0) {
    int run = 0, first = 0;
    if (lane < E) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w % RW == 0) run = s_off[lane] + s_ub[w][lane];
        if (w == 0) first = run;
        s_base[w][lane] = run;
        run += __popcll(s_col[w][lane]);
      }
    }
    const int n = lane < E ? run - first : 0;  // this tile's tokens of expert lane
    const int incl = wave_incl_scan(n, lane);
    if (lane < E) s_run[lane] = incl - n;
    s_dl[lane] = lane < E ? first - (incl - n) : 0;
    if (lane == 63) s_run[64] = incl;
  }
  __syncthreads();
  if (t < L) {
    for (int k = 0; k < K; ++k) {
      int pos = -1;  // (a mask with fewer than K bits leaves -1)
      if (m != 0) {
        const int e = lowest_bit(m);
        m &= m - 1;
        const uint64_t ce = s_col[wave][e];
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(ce >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)ce, 0));
        pos = s_base[wave][e] + below;
        const int lp = s_run[e] + (s_base[wave][e] - s_base[0][e]) + below;
        if (lp < MAXE) {  // always true when the masks hold K bits each
          s_tok[lp] = (int32_t)t;
          s_ex[lp] = (uint8_t)e;
        }
      }
      s_tim[tid * K + k] = pos;
    }
  }
  __syncthreads();
  // The staged values are read (indices clamped into the arrays) before any
  // store goes out, so the LDS reads do not wait on each other behind the
  // stores' bounds branches.
  constexpr int NJ = MAXE / 256;
  const int n = min(s_run[64], MAXE);
  const int64_t R = L * K;
  int pv[NJ], tv[NJ];
#pragma unroll
  for (int u = 0; u < NJ; ++u) {
    const int j = min(tid + u * 256, MAXE - 1);
    pv[u] = j + s_dl[s_ex[j] & 63];  // entries past n are not stored
    tv[u] = s_tok[j];
  }
#pragma unroll
  for (int u = 0; u < NJ; ++u)  // pos < R always holds when the masks hold K bits each
    if (tid + u * 256 < n && pv[u] < R) eti[pv[u]] = tv[u];
  // rows t0 .. t0 + 255 of token_index_map are one contiguous run
  const int64_t t0 = (int64_t)tile * 256;
  const int nt = (int)min((int64_t)256, L - t0) * K;
  int mv[NJ];
#pragma unroll
  for (int u = 0; u < NJ; ++u) mv[u] = s_tim[min(tid + u * 256, MAXE - 1)];
#pragma unroll
  for (int u = 0; u < NJ; ++u)
    if (tid + u * 256 < nt) tim[t0 * K + tid + u * 256] = mv[u];
}

// ---------------------------------------------------------------- wide E
// Bit-form map for 64 < E <= 64 P (P = 2, 4, 8 or 16 words of 64 experts per
// token), K <= 8.  Same outputs as the E <= 64 kernels, per 64-token part:
// each token's expert mask as P words (word q = experts 64q .. 64q+63), the
// part's column ballot of every expert and the part's per-expert counts.
//
// Step 1.  One wavefront per workgroup routes one part in P rounds of 64 / P
// tokens, P lanes per token: lane q of a token owns experts 64q .. 64q+63.
// A round's logit rows (one contiguous run of 16 KB at most) are copied into
// LDS with 1 KB direct-to-LDS transfers.  As in the E <= 64 router, each lane
// reads its slice from LDS twice, 4 values at a time, starting at a
// lane-dependent chunk (bank spreading), so few registers are live and many
// workgroups share a CU: pass 1 keeps the slice's KM largest values (med3
// network), the token's P lists are merged by a butterfly of shuffles, which
// gives every lane of the token the token's K largest values and so the
// K-th value thr; pass 2 marks the slice's experts >= thr.  Surplus marks can
// only be ties with thr and are dropped from the highest expert ids (highest
// lane first); a shortfall (NaN logits, outside the contract) is filled with
// the lowest unmarked ids, so every token gets exactly K valid experts.
// Slots follow the lanes' order, hence ascending expert id.  The part's
// masks collect in LDS as [token][word]; after the last round a bit transpose
// of each word across the wavefront gives the part's columns.
template <int P, int KM, bool VEC>
__global__ __launch_bounds__(64) void k1_route_wide_mask(
    const float* __restrict__ logits, int64_t L, int E, int K, int64_t NP,
    int32_t* __restrict__ tei, float* __restrict__ gates, uint64_t* __restrict__ tmask,
    uint64_t* __restrict__ tcol, int32_t* __restrict__ partcnt) {
  constexpr int TPR = 64 / P;                  // tokens per round
  constexpr int STAGEB = 16384 + (VEC ? 0 : 1024);
  __shared__ __attribute__((aligned(16))) char stage[STAGEB];
  __shared__ uint64_t smask[64][P];
  const int lane = threadIdx.x;
  const int q = lane % P;               // slice of the token
  const int i = lane / P;               // token of the round
  const int grp = lane - q;             // first lane of the token
  const int e0 = 64 * q;
  const int ne = max(0, min(64, E - e0));  // experts in this lane's slice
  const uint64_t valid = ne >= 64 ? ~0ull : ((1ull << ne) - 1);
  const int rot = lane & 15;
  const int rowb = 4 * E;
  int64_t part;
  {  // contiguous runs of parts per XCD: neighbouring parts' count words meet in one L2
    const int64_t nb = gridDim.x, b = blockIdx.x, qq = nb >> 3, r = nb & 7, x = b & 7;
    part = x * qq + (x < r ? x : r) + (b >> 3);
  }
  RouteSrc src;
  {
    const char* lbase = reinterpret_cast<const char*>(logits);
    src.mis = (int64_t)(reinterpret_cast<uintptr_t>(lbase) & 15);  // 0 when VEC
    src.abase = lbase - src.mis;
    src.end16 = (src.mis + L * rowb + 15) & ~(int64_t)15;
  }
  // E == 64 P (every lane owns 64 experts) with 16-byte aligned rows and
  // L >= TPR: a round is exactly 16 KB, read through registers (sixteen
  // coalesced 16-byte loads per lane) and written to LDS by the wavefront;
  // the last round reads rows [L - TPR, L) so every load is in range.
  // Otherwise direct-to-LDS copies.
  const bool regpath = VEC && E == 64 * P && L >= TPR;
  for (int rd = 0; rd < P; ++rd) {
    const int64_t tr0 = part * 64 + (int64_t)rd * TPR;   // first token of the round
    const int64_t t = tr0 + i;
    const bool live = t < L;
    const float* row;
    if (regpath) {
      typedef float v4f __attribute__((ext_vector_type(4)));
      const int64_t fr = min(tr0, L - TPR);  // first row of the round's copy
      const v4f* pb = reinterpret_cast<const v4f*>(logits) + fr * (E >> 2);  // uniform
      v4f vv[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) vv[c] = __builtin_nontemporal_load(pb + c * 64 + lane);
      // (the previous round's LDS reads come first in program order)
#pragma unroll
      for (int c = 0; c < 16; ++c) reinterpret_cast<v4f*>(stage)[c * 64 + lane] = vv[c];
      __builtin_amdgcn_wave_barrier();
      const int srow = (int)min<int64_t>(t - fr, TPR - 1);  // rows past L: any row
      row = reinterpret_cast<const float*>(stage + (int64_t)srow * rowb) + e0;
    } else {
      const int64_t first = src.mis + tr0 * rowb;
      const int64_t first16 = first & ~(int64_t)15;
      const int delta = (int)(first - first16);
      const int nq = tr0 < L ? (int)((delta + (int64_t)TPR * rowb + 1023) >> 10) : 0;
      // the previous round's LDS reads are done before its stage is rewritten
      __builtin_amdgcn_s_waitcnt(0);
      for (int c = 0; c < nq; ++c) {
        const int64_t off = first16 + (int64_t)c * 1024 + lane * 16;
        const char* g = src.abase + (off + 16 <= src.end16 ? off : 0);
        __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(stage + c * 1024), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      row = reinterpret_cast<const float*>(stage + delta + (int64_t)i * rowb) + e0;
    }
    auto chunk = [&](int c, float (&v)[4]) {
      if (VEC && 4 * c + 4 <= ne) {
        const float4 x = reinterpret_cast<const float4*>(row)[c];
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = 4 * c + u < ne ? row[4 * c + u] : -INFINITY;
      }
    };
    float b[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) b[k] = -INFINITY;
    // (not unrolled: four values live at a time keep the register count low)
#pragma unroll 2
    for (int j = 0; j < 16; ++j) {
      float v[4];
      chunk((j + rot) & 15, v);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int k = KM - 1; k > 0; --k) b[k] = __builtin_amdgcn_fmed3f(b[k - 1], b[k], v[u]);
        b[0] = fmaxf(b[0], v[u]);
      }
    }
#pragma unroll
    for (int o = 1; o < P; o <<= 1) {
      float pb[KM];
#pragma unroll
      for (int k = 0; k < KM; ++k) pb[k] = __shfl_xor(b[k], o);
#pragma unroll
      for (int j = 0; j < KM; ++j) {
#pragma unroll
        for (int k = KM - 1; k > 0; --k) b[k] = __builtin_amdgcn_fmed3f(b[k - 1], b[k], pb[j]);
        b[0] = fmaxf(b[0], pb[j]);
      }
    }
    float thr = b[0];
#pragma unroll
    for (int k = 1; k < KM; ++k) thr = (k == K - 1) ? b[k] : thr;

    uint64_t ge = 0, gt = 0;
#pragma unroll 2
    for (int j = 0; j < 16; ++j) {
      const int c = (j + rot) & 15;
      float v[4];
      chunk(c, v);
      const uint32_t g4 = (v[0] >= thr ? 1u : 0u) | (v[1] >= thr ? 2u : 0u) |
                          (v[2] >= thr ? 4u : 0u) | (v[3] >= thr ? 8u : 0u);
      const uint32_t t4 = (v[0] > thr ? 1u : 0u) | (v[1] > thr ? 2u : 0u) |
                          (v[2] > thr ? 4u : 0u) | (v[3] > thr ? 8u : 0u);
      ge |= (uint64_t)g4 << (4 * c);
      gt |= (uint64_t)t4 << (4 * c);
    }
    ge &= valid;
    gt &= valid;
    int cnt[P], tie[P];
    const int mycnt = __builtin_popcountll(ge), mytie = __builtin_popcountll(ge & ~gt);
#pragma unroll
    for (int r = 0; r < P; ++r) {
      cnt[r] = __shfl(mycnt, grp + r);
      tie[r] = __shfl(mytie, grp + r);
    }
    int total = 0, above = 0;
#pragma unroll
    for (int r = 0; r < P; ++r) {
      total += cnt[r];
      above += r > q ? tie[r] : 0;
    }
    if (total > K) {  // drop surplus ties from the highest ids
      int drop = min(max(total - K - above, 0), mytie);
      uint64_t ties = ge & ~gt;
      for (; drop > 0; --drop) {
        const int hb = 63 - __builtin_clzll(ties);
        ties &= ~(1ull << hb);
        ge &= ~(1ull << hb);
      }
    } else if (total < K) {  // NaN logits only: fill with the lowest free ids
      const int myfree = __builtin_popcountll(valid & ~ge);
      int below = 0;
#pragma unroll
      for (int r = 0; r < P; ++r) {
        const int fr = __shfl(myfree, grp + r);
        below += r < q ? fr : 0;
      }
      int add = min(max(K - total - below, 0), myfree);
      uint64_t fr = valid & ~ge;
      for (; add > 0; --add) {
        const uint64_t lo = fr & (~fr + 1);
        fr &= ~lo;
        ge |= lo;
      }
    }
    const int kept = __builtin_popcountll(ge);
    int base = 0;
#pragma unroll
    for (int r = 0; r < P; ++r) {
      const int kr = __shfl(kept, grp + r);
      base += r < q ? kr : 0;
    }
    const uint64_t m = live ? ge : 0ull;
    smask[rd * TPR + i][q] = m;
    if (live) {
      tmask[t * P + q] = m;
      const float vmax = b[0];
      float ssum = 0.f;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (k < K) ssum += expf(b[k] - vmax);
      const float inv = 1.0f / ssum;
      uint64_t mm = m;
      for (int slot = base; mm != 0 && slot < K; ++slot) {
        const int j = __builtin_ctzll(mm);
        mm &= mm - 1;
        tei[t * K + slot] = e0 + j;
        gates[t * K + slot] = expf(row[j] - vmax) * inv;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // columns: word qw of the part's 64 tokens, transposed -> expert 64 qw + lane
  for (int qw = 0; qw < P; ++qw) {
    const uint64_t mycol = wave_transpose64(smask[lane][qw], lane);
    const int e = 64 * qw + lane;
    if (e < E) {
      tcol[part * E + e] = mycol;
      partcnt[(int64_t)e * NP + part] = __popcll(mycol);
    }
  }
}

// Step 3 for the wide bit form (E <= 64 W): one workgroup per 256-token tile
// (four parts, one token per thread).  As in the E <= 64 scatter, a route's
// position is the expert's segment start plus the tile base from the scan,
// plus the part's running base inside the tile, plus the set bits of the
// part's column below the token's lane; the tile's entries are staged in
// LDS by expert and written out run by run, and the tile's token_index_map
// rows leave as one contiguous run.  Expert-indexed work (segment starts,
// running bases, run starts) is spread over the 256 threads, EPT
// consecutive experts each.
template <int W, int KMAX>
__global__ __launch_bounds__(256) void k3_scatter_wide(const uint64_t* __restrict__ tmask,
                                                       const uint64_t* __restrict__ tcol,
                                                       int64_t L, int E, int K, int NU,
                                                       const int32_t* __restrict__ unitbase,
                                                       const int32_t* __restrict__ total,
                                                       int32_t* __restrict__ eti,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tim) {
  constexpr int EM = 64 * W;
  constexpr int EPT = (EM + 255) / 256;  // experts per thread
  constexpr int MAXE = 256 * KMAX;       // entries of one tile (K <= KMAX), sized as in k3_scatter_mask
  static_assert((EM & (EM - 1)) == 0, "expert ids of staged entries are masked with EM - 1");
  __shared__ int s_off[EM + 1];
  __shared__ int scratch[4];
  __shared__ uint64_t s_col[4][EM];
  __shared__ int s_base[4][EM];
  __shared__ int s_run[EM + 1];
  __shared__ int s_tok[MAXE];
  // expert of each staged entry: the entry's position in
  // expert_token_indices is its index plus s_base[0][e] - s_run[e]
  __shared__ uint16_t s_ex[MAXE];
  __shared__ int s_tim[MAXE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int tile;
  {
    const int nb = gridDim.x, b = blockIdx.x, q = nb >> 3, r = nb & 7, x = b & 7;
    tile = x * q + (x < r ? x : r) + (b >> 3);
  }
  const int64_t t = (int64_t)tile * 256 + tid;
  uint64_t mk[W];
#pragma unroll
  for (int qw = 0; qw < W; ++qw) mk[qw] = t < L ? tmask[t * W + qw] : 0ull;
  for (int f = tid; f < 4 * EM; f += 256) {
    const int w = f / EM, e = f % EM;
    const int64_t part = (int64_t)tile * 4 + w;
    s_col[w][e] = (e < E && part * 64 < L) ? tcol[part * E + e] : 0ull;
  }
  // expert segment starts: exclusive scan of the totals
  int tv[EPT], ub[EPT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    tv[j] = e < E ? total[e] : 0;
    ub[j] = e < E ? unitbase[(int64_t)e * NU + tile] : 0;
    sum += tv[j];
  }
  int tot;
  int ex = block256_incl_scan(sum, scratch, &tot) - sum;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    if (e < E) s_off[e] = ex;
    ex += tv[j];
  }
  if (tid == 0) s_off[E] = tot;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += 256) offsets[e] = s_off[e];
  // running bases of the four parts and the tile's count of each expert
  int n[EPT];
  int nsum = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    n[j] = 0;
    if (e < E) {
      int run = s_off[e] + ub[j];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s_base[w][e] = run;
        const int c = __popcll(s_col[w][e]);
        run += c;
        n[j] += c;
      }
    }
    nsum += n[j];
  }
  int ntot;
  int rx = block256_incl_scan(nsum, scratch, &ntot) - nsum;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid * EPT + j;
    if (e < E) s_run[e] = rx;
    rx += n[j];
  }
  if (tid == 0) s_run[E] = ntot;
  __syncthreads();
  if (t < L) {
    int qw = 0;
    for (int k = 0; k < K; ++k) {
      int pos = -1;  // (masks with fewer than K bits leave -1)
      while (qw < W && mk[qw] == 0) ++qw;
      if (qw < W) {
        const int e = 64 * qw + lowest_bit(mk[qw]);
        mk[qw] &= mk[qw] - 1;
        const uint64_t ce = s_col[wave][e];
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(ce >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)ce, 0));
        pos = s_base[wave][e] + below;
        const int lp = s_run[e] + (s_base[wave][e] - s_base[0][e]) + below;
        if (lp < MAXE) {  // always true when the masks hold K bits each
          s_tok[lp] = (int32_t)t;
          s_ex[lp] = (uint16_t)e;
        }
      }
      s_tim[tid * K + k] = pos;
    }
  }
  __syncthreads();
  constexpr int NJ = MAXE / 256;
  const int nrun = min(s_run[E], MAXE);
  const int64_t R = L * K;
  int pv[NJ], tk[NJ];
#pragma unroll
  for (int u = 0; u < NJ; ++u) {
    const int j = min(tid + u * 256, MAXE - 1);
    const int e = s_ex[j] & (EM - 1);  // entries past nrun are not stored
    pv[u] = j + s_base[0][e] - s_run[e];
    tk[u] = s_tok[j];
  }
#pragma unroll
  for (int u = 0; u < NJ; ++u)  // pos < R always holds when the masks hold K bits each
    if (tid + u * 256 < nrun && pv[u] >= 0 && pv[u] < R) eti[pv[u]] = tk[u];
  const int64_t t0 = (int64_t)tile * 256;
  const int nt = (int)min((int64_t)256, L - t0) * K;
  int mv[NJ];
#pragma unroll
  for (int u = 0; u < NJ; ++u) mv[u] = s_tim[min(tid + u * 256, MAXE - 1)];
#pragma unroll
  for (int u = 0; u < NJ; ++u)
    if (tid + u * 256 < nt) tim[t0 * K + tid + u * 256] = mv[u];
}

// Exclusive scan of each row of a [rows][C] count table (one workgroup per
// row): base[r][c] = r * row_offset + sum of counts[r][0..c).  total[r] gets
// the row sum when total is not null.  With G > 1 the input rows hold G
// consecutive counts per entry ([rows][C * G]), which are added first.
// A pass covers V rounds of 256 consecutive entries, one entry per thread
// and round, so that loads and stores are contiguous across lanes; each
// wavefront scans its 64 entries of a round, and one barrier per pass
// shares the 4 V wavefront sums, scanned in (round, wavefront) order.
template <int G>
__global__ __launch_bounds__(256) void seg_scan(const int32_t* __restrict__ cnt, int C,
                                                int64_t row_offset, int32_t* __restrict__ base,
                                                int32_t* __restrict__ total) {
  constexpr int V = 16;  // rounds per pass; V * 4 wavefront sums == one wavefront
  static_assert(V * 4 == kWave, "one lane per wavefront sum");
  __shared__ int s_w[V * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x;
  const int32_t* in = cnt + (int64_t)r * C * G;
  int32_t* out = base + (int64_t)r * C;
  int run = 0;
  for (int c0 = 0; c0 < C; c0 += 256 * V) {
    // Every load goes out before any is used: entries past C read entry
    // C - 1 (a branch around each load would make each wait for the last).
    int x[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c = c0 + j * 256 + threadIdx.x;
      const int64_t cc = c < C ? c : C - 1;
      int v = 0;
      if constexpr (G == 4) {
        const int4 q = *reinterpret_cast<const int4*>(in + cc * 4);
        v = q.x + q.y + q.z + q.w;
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) v += in[cc * G + g];
      }
      x[j] = c < C ? v : 0;
    }
    int ex[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int inc = wave_incl_scan(x[j], lane);
      ex[j] = inc - x[j];
      if (lane == 63) s_w[j * 4 + wave] = inc;
    }
    __syncthreads();
    const int wv = s_w[lane];
    const int wex = wave_incl_scan(wv, lane) - wv;  // before (round, wave) = lane
    const int ptot = __builtin_amdgcn_readlane(wex + wv, 63);
    const int64_t add = r * row_offset + run;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c = c0 + j * 256 + threadIdx.x;
      const int before = __builtin_amdgcn_readlane(wex, j * 4 + wave);  // wave-uniform lane
      if (c < C) out[c] = (int32_t)(add + before + ex[j]);
    }
    run += ptot;
    __syncthreads();  // s_w is rewritten by the next pass
  }
  if (total != nullptr && threadIdx.x == 0) total[r] = run;
}

// Step 3: per tile, scan each expert's map row segment and scatter.
// A row segment is T bytes = T/16 lanes of 16 bytes, so one wavefront
// covers 64/(T/16) rows per pass; the wavefront issues the loads of U passes
// before scanning any of them.
__global__ __launch_bounds__(256) void k3_scatter(const uint8_t* __restrict__ map, int64_t Lpad,
                                                  int E, int K, int T, int C,
                                                  const int32_t* __restrict__ tilebase,
                                                  const int32_t* __restrict__ total,
                                                  int32_t* __restrict__ eti,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ tim) {
  __shared__ int s_off[257];
  __shared__ int scratch[4];
  const int tid = threadIdx.x;
  const int v = tid < E ? total[tid] : 0;
  int tot;
  const int inc = block256_incl_scan(v, scratch, &tot);
  if (tid < E) s_off[tid] = inc - v;
  if (tid == 0) s_off[E] = tot;
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) offsets[tid] = s_off[tid];
    if (tid == 0) offsets[E] = s_off[E];
  }

  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * T;
  const int lane = tid & 63, wave = tid >> 6;
  const int seg = T >> 4;            // lanes per row (16, 32 or 64)
  const int rpw = 64 / seg;          // rows per wavefront pass
  const int sub = lane / seg, sl = lane % seg;
  constexpr int U = 4;
  for (int e0 = wave * rpw; e0 < E; e0 += 4 * rpw * U) {
    uint4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * 4 * rpw + sub;
      const bool ok = e < E;
      const uint4 w = *reinterpret_cast<const uint4*>(map + (int64_t)(ok ? e : 0) * Lpad + t0 +
                                                      sl * 16);
      q[u] = ok ? w : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * 4 * rpw + sub;
      const int cnt = nonzero_bytes(q[u].x) + nonzero_bytes(q[u].y) + nonzero_bytes(q[u].z) +
                      nonzero_bytes(q[u].w);
      int incl = cnt;
      for (int o = 1; o < seg; o <<= 1) {
        const int x = __shfl_up(incl, o, seg);
        if (sl >= o) incl += x;
      }
      if (e < E && cnt > 0) {
        int pos = s_off[e] + tilebase[(int64_t)e * C + tile] + incl - cnt;
        const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const uint32_t val = (w[b >> 2] >> ((b & 3) * 8)) & 0xffu;
          if (val) {
            const int64_t t = t0 + sl * 16 + b;
            eti[pos] = (int32_t)t;
            tim[t * K + (val - 1)] = pos;
            ++pos;
          }
        }
      }
    }
  }
}

void launch_seg_scan(const int32_t* cnt, int rows, int C, int64_t row_offset, int32_t* base,
                     int32_t* total, hipStream_t s) {
  hipLaunchKernelGGL(seg_scan<1>, dim3(rows), dim3(256), 0, s, cnt, C, row_offset, base, total);
}

// The bit-form kernels (256-token tiles) serve E <= 1024 and K <= 8: one
// 64-bit mask word per token for E <= 64, P (a power of two, 2..16) words
// for larger E.  K > 8 (E <= 256) uses the byte map with 256..1024-token
// tiles.
static bool stream_path(int E, int K) { return E <= 1024 && K <= 8; }

static int mask_words(int E) {
  if (E <= 64) return 1;
  int P = 2;
  while (64 * P < E) P <<= 1;
  return P;
}

DispatchPlan plan_dispatch(int64_t L, int E, int K) {
  DispatchPlan p;
  p.stream = stream_path(E, K);
  p.W = p.stream ? mask_words(E) : 0;
  int T;
  if (p.stream) {
    T = 256;
  } else {
    // T is a power of two in [256, 1024] (the scatter kernel splits a
    // wavefront into T/16-lane row segments), with E * T <= 32 KB of LDS
    // where possible (E * T <= 64 KB always, since E <= 256).
    T = 1024;
    while (T > 256 && E * T > 32768) T >>= 1;
  }
  p.T = T;
  p.C = (int)((L + T - 1) / T);
  p.Lpad = (int64_t)p.C * T;
  // every part of every 256-token tile is routed (parts past L write zero
  // counts), so the grouped scan reads only written entries
  p.NP = p.stream ? (int64_t)4 * p.C : 0;
  // map: W 64-bit expert mask words per token (bit form) or the [E][Lpad] byte map
  const size_t map_bytes = p.stream ? (size_t)8 * p.W * p.Lpad : (size_t)E * p.Lpad;
  size_t o = 0;
  p.off_map = o;   o = align_up(o + map_bytes, 256);
  p.off_col = o;   o = align_up(o + (p.stream ? (size_t)8 * E * (p.Lpad / 64) : 0), 256);
  p.off_cnt = o;   o = align_up(o + (size_t)E * (p.stream ? 4 * p.C : p.C) * 4, 256);
  p.off_base = o;  o = align_up(o + (size_t)E * p.C * 4, 256);
  p.off_total = o; o = align_up(o + (size_t)(E > 256 ? E : 256) * 4, 256);
  p.bytes = o;
  return p;
}

template <int G>
static void launch_k1(const DispatchPlan& pl, int64_t L, int E, int K, const float* logits,
                      int32_t* tei, float* gates, uint8_t* map, int32_t* cnt, hipStream_t s) {
  const bool vec4 = (E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  if (vec4)
    hipLaunchKernelGGL((k1_route_map<G, true>), dim3(pl.C), dim3(256), (size_t)E * pl.T, s, logits,
                       L, E, K, pl.T, pl.C, pl.Lpad, tei, gates, map, cnt);
  else
    hipLaunchKernelGGL((k1_route_map<G, false>), dim3(pl.C), dim3(256), (size_t)E * pl.T, s,
                       logits, L, E, K, pl.T, pl.C, pl.Lpad, tei, gates, map, cnt);
}


hipError_t launch_dispatch(const DispatchPlan& pl, int64_t L, int E, int K, const float* logits,
                           int32_t* eti, int32_t* offsets, int32_t* tei, int32_t* tim,
                           float* gates, char* ws, hipStream_t s) {
  uint8_t* map = reinterpret_cast<uint8_t*>(ws + pl.off_map);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + pl.off_cnt);
  int32_t* base = reinterpret_cast<int32_t*>(ws + pl.off_base);
  int32_t* total = reinterpret_cast<int32_t*>(ws + pl.off_total);
  {
    LaunchTimer lt("dispatch_route_map", s);
    const int q = (E + 3) / 4;  // lanes needed per token
    const bool rows_ok = (E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
    if (pl.stream) {
      uint64_t* tmask = reinterpret_cast<uint64_t*>(ws + pl.off_map);
      uint64_t* tcol = reinterpret_cast<uint64_t*>(ws + pl.off_col);
#define K1M(EBV, KV, VV)                                                                        \
  if (VV && EBV == 64 && E == 64 && L >= 64)                                                    \
    hipLaunchKernelGGL((k1_route_mask64<KV>), dim3(pl.NP), dim3(64), 0, s, logits, L, E, K,       \
                       pl.NP, tei, gates, tmask, tcol, cnt);                                    \
  else                                                                                          \
    hipLaunchKernelGGL((k1_route_mask<EBV, KV, VV>), dim3(pl.NP), dim3(64), 0, s, logits, L, E,   \
                       K, pl.NP, tei, gates, tmask, tcol, cnt)
#define K1M_K(EBV)                                                                              \
  if (!rows_ok) {                                                                               \
    K1M(EBV, 8, false);                                                                         \
  } else {                                                                                      \
    switch (K) {                                                                                \
      case 1: K1M(EBV, 1, true); break;                                                         \
      case 2: K1M(EBV, 2, true); break;                                                         \
      case 3: K1M(EBV, 3, true); break;                                                         \
      case 4: K1M(EBV, 4, true); break;                                                         \
      case 5: K1M(EBV, 5, true); break;                                                         \
      case 6: K1M(EBV, 6, true); break;                                                         \
      case 7: K1M(EBV, 7, true); break;                                                         \
      default: K1M(EBV, 8, true); break;                                                        \
    }                                                                                           \
  }
      if (E <= 16) {
        K1M_K(16)
      } else if (E <= 32) {
        K1M_K(32)
      } else if (E <= 64) {
        K1M_K(64)
      } else {
#define K1W(PV, KV, VV)                                                                         \
  hipLaunchKernelGGL((k1_route_wide_mask<PV, KV, VV>), dim3(pl.NP), dim3(64), 0, s, logits, L, E, \
                     K, pl.NP, tei, gates, tmask, tcol, cnt)
#define K1W_K(PV)                                                                               \
  if (!rows_ok) {                                                                               \
    K1W(PV, 8, false);                                                                          \
  } else {                                                                                      \
    switch (K) {                                                                                \
      case 1: K1W(PV, 1, true); break;                                                          \
      case 2: K1W(PV, 2, true); break;                                                          \
      case 3: K1W(PV, 3, true); break;                                                          \
      case 4: K1W(PV, 4, true); break;                                                          \
      case 5: K1W(PV, 5, true); break;                                                          \
      case 6: K1W(PV, 6, true); break;                                                          \
      case 7: K1W(PV, 7, true); break;                                                          \
      default: K1W(PV, 8, true); break;                                                         \
    }                                                                                           \
  }
        switch (pl.W) {
          case 2: K1W_K(2) break;
          case 4: K1W_K(4) break;
          case 8: K1W_K(8) break;
          default: K1W_K(16) break;
        }
#undef K1W_K
#undef K1W
      }
#undef K1M_K
#undef K1M
    } else if (rows_ok && E <= 64) {
      const size_t sh = (size_t)E * pl.T;
#define MOE_K1R(EVV)                                                                            \
  hipLaunchKernelGGL((k1_route_map_rows<EVV>), dim3(pl.C), dim3(256), sh, s, logits, L, E, K,   \
                     pl.T, pl.C, pl.Lpad, tei, gates, map, cnt)
      if (E <= 8) MOE_K1R(8);
      else if (E <= 16) MOE_K1R(16);
      else if (E <= 32) MOE_K1R(32);
      else MOE_K1R(64);
#undef MOE_K1R
    } else if (q <= 1) launch_k1<1>(pl, L, E, K, logits, tei, gates, map, cnt, s);
    else if (q <= 2) launch_k1<2>(pl, L, E, K, logits, tei, gates, map, cnt, s);
    else if (q <= 4) launch_k1<4>(pl, L, E, K, logits, tei, gates, map, cnt, s);
    else if (q <= 8) launch_k1<8>(pl, L, E, K, logits, tei, gates, map, cnt, s);
    else if (q <= 16) launch_k1<16>(pl, L, E, K, logits, tei, gates, map, cnt, s);
    else if (q <= 32) launch_k1<32>(pl, L, E, K, logits, tei, gates, map, cnt, s);
    else launch_k1<64>(pl, L, E, K, logits, tei, gates, map, cnt, s);
  }
  {
    LaunchTimer lt("dispatch_expert_scan", s);
    if (pl.stream)  // per-part counts, added four at a time into 256-token tiles
      hipLaunchKernelGGL(seg_scan<4>, dim3(E), dim3(256), 0, s, cnt, pl.C, (int64_t)0, base,
                         total);
    else
      launch_seg_scan(cnt, E, pl.C, 0, base, total, s);
  }
  {
    LaunchTimer lt("dispatch_scatter", s);
    const uint64_t* tmask = reinterpret_cast<const uint64_t*>(ws + pl.off_map);
    const uint64_t* tcol = reinterpret_cast<const uint64_t*>(ws + pl.off_col);
#define K3WK(WV, KX)                                                                            \
  hipLaunchKernelGGL((k3_scatter_wide<WV, KX>), dim3(pl.C), dim3(256), 0, s, tmask, tcol, L, E, K, \
                     pl.C, base, total, eti, offsets, tim)
#define K3W(WV)                                                                                 \
  do {                                                                                          \
    if (K <= 2) K3WK(WV, 2);                                                                    \
    else if (K <= 4) K3WK(WV, 4);                                                               \
    else if (K <= 6) K3WK(WV, 6);                                                               \
    else K3WK(WV, 8);                                                                           \
  } while (0)
#define K3M(KX)                                                                                 \
  hipLaunchKernelGGL((k3_scatter_mask<4, KX>), dim3(pl.C), dim3(256), 0, s, tmask, tcol, L, E, K,  \
                     pl.C, base, total, eti, offsets, tim)
    if (pl.stream && pl.W == 1) {
      if (K <= 2) K3M(2);
      else if (K <= 4) K3M(4);
      else if (K <= 6) K3M(6);
      else K3M(8);
    }
    else if (pl.stream && pl.W == 2)
      K3W(2);
    else if (pl.stream && pl.W == 4)
      K3W(4);
    else if (pl.stream && pl.W == 8)
      K3W(8);
    else if (pl.stream)
      K3W(16);
#undef K3W
#undef K3WK
#undef K3M
    else
      hipLaunchKernelGGL(k3_scatter, dim3(pl.C), dim3(256), 0, s, map, pl.Lpad, E, K, pl.T, pl.C,
                         base, total, eti, offsets, tim);
  }
  return hipGetLastError();
}

}  // namespace moe
