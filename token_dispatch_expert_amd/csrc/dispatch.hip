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
// come from group reductions and a group prefix count.
template <int G>
__device__ __forceinline__ void route_token(const float (&v)[4], int lg, int E, int K, int64_t t,
                                            int tl, int T, int32_t* __restrict__ tei,
                                            float* __restrict__ gates, uint8_t* smap) {
  int ev[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ev[j] = lg * 4 + j;
  unsigned sel = 0;
  float vmax = 0.f;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = INT_MAX;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool cand = !((sel >> j) & 1u) && ev[j] < E;
      if (cand && (v[j] > bv || (v[j] == bv && ev[j] < be))) {
        bv = v[j];
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

template <int EB> struct MaskT { using type = uint32_t; };
template <> struct MaskT<64> { using type = uint64_t; };

__device__ __forceinline__ int lowest_bit(uint32_t m) { return __builtin_ctz(m); }
__device__ __forceinline__ int lowest_bit(uint64_t m) { return __builtin_ctzll(m); }
__device__ __forceinline__ int bit_count(uint32_t m) { return __builtin_popcount(m); }
__device__ __forceinline__ int bit_count(uint64_t m) { return __builtin_popcountll(m); }

// Step 1, streaming form for E <= EB (E % 4 == 0, EB in {16, 32, 64}) and a
// compile-time K <= 8: one tile of 256 tokens per workgroup, one token per
// lane.  Each wavefront copies the 64 consecutive logit rows of its tokens
// (one contiguous run of 256 E bytes) straight into LDS with 1 KB
// global_load_lds transfers; each lane then reads its own row back, starting
// at a lane-dependent 16-byte chunk so that the lanes of one LDS cycle hit
// different banks.
//
// Selection is exact top-K with ties to the lower expert id, done in two
// passes over the row instead of a K-step arg-max:
//   pass 1 keeps the K largest values as a descending register list; a new
//          value x enters as b[0] = max(b[0], x), b[i] = med3(b[i-1], b[i], x)
//          (one instruction per slot, no index bookkeeping);
//   pass 2 marks every expert whose logit is >= b[K-1] in a bit mask.
// The mask has at least K bits; extra bits can only be ties with b[K-1], and
// dropping those of the highest ids leaves the lower-id choice.  Slots are the
// mask bits in ascending id order.  NaN logits (outside the contract) cannot
// produce an invalid id: the mask is trimmed or filled to exactly K bits.
template <int EB, int K>
__global__ __launch_bounds__(256) void k1_route_map_stream(const float* __restrict__ logits,
                                                           int64_t L, int E, int C, int64_t Lpad,
                                                           int32_t* __restrict__ tei,
                                                           float* __restrict__ gates,
                                                           uint8_t* __restrict__ map,
                                                           int32_t* __restrict__ tilecnt) {
  using mask_t = typename MaskT<EB>::type;
  constexpr int T = 256;
  __shared__ __attribute__((aligned(16))) char stage[T * 4 * EB];  // 256 rows of 4 E bytes
  __shared__ __attribute__((aligned(16))) uint8_t smap[EB * T];     // [E][T] slot + 1
  const int tile = blockIdx.x;
  const int64_t t0 = (int64_t)tile * T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rowb = 4 * E;

  {  // this wavefront's 64 rows are contiguous in memory
    const int64_t first = (t0 + wave * 64) * rowb;
    const int64_t total = L * rowb;
    char* dst = stage + wave * 64 * rowb;
    const int nq = E >> 2;  // 64 rows x 4 E bytes = E/4 transfers of 1 KB
    for (int q = 0; q < nq; ++q) {
      const int64_t off = first + q * 1024 + lane * 16;
      const char* g = reinterpret_cast<const char*>(logits) + (off + 16 <= total ? off : 0);
      __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(dst + q * 1024), 16, 0, 0);
    }
  }
  for (int i = threadIdx.x; i < (E * T) >> 4; i += 256)
    reinterpret_cast<uint4*>(smap)[i] = make_uint4(0, 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int tl = wave * 64 + lane;
  const int64_t t = t0 + tl;
  if (t < L) {
    const float* row = reinterpret_cast<const float*>(stage + tl * rowb);
    const int nc = E >> 2;
    const int rot = lane % nc;

    float b[K];
#pragma unroll
    for (int i = 0; i < K; ++i) b[i] = -INFINITY;
    for (int j = 0, c = rot; j < nc; ++j, c = (c + 1 == nc) ? 0 : c + 1) {
      const float4 q = reinterpret_cast<const float4*>(row)[c];
      const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float x = qv[u];
#pragma unroll
        for (int i = K - 1; i > 0; --i) b[i] = __builtin_amdgcn_fmed3f(b[i - 1], b[i], x);
        b[0] = fmaxf(b[0], x);
      }
    }
    const float thr = b[K - 1];

    mask_t m = 0;
    for (int j = 0, c = rot; j < nc; ++j, c = (c + 1 == nc) ? 0 : c + 1) {
      const float4 q = reinterpret_cast<const float4*>(row)[c];
      const mask_t m4 = (q.x >= thr ? 1u : 0u) | (q.y >= thr ? 2u : 0u) | (q.z >= thr ? 4u : 0u) |
                        (q.w >= thr ? 8u : 0u);
      m |= m4 << (4 * c);
    }
    int cnt = bit_count(m);
    for (int e = E - 1; e >= 0 && cnt > K; --e) {
      if (((m >> e) & 1) && !(row[e] > thr)) {
        m &= ~((mask_t)1 << e);
        --cnt;
      }
    }
    for (int e = 0; e < E && cnt < K; ++e) {
      if (!((m >> e) & 1)) {
        m |= (mask_t)1 << e;
        ++cnt;
      }
    }

    const float vmax = b[0];
    float ssum = 0.f;
#pragma unroll
    for (int i = 0; i < K; ++i) ssum += expf(b[i] - vmax);
    const float inv = 1.0f / ssum;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = lowest_bit(m);
      m &= m - 1;
      tei[t * K + k] = e;
      gates[t * K + k] = expf(row[e] - vmax) * inv;
      smap[e * T + tl] = (uint8_t)(k + 1);
    }
  }
  __syncthreads();

  const int nv = T >> 4;
  for (int e = wave; e < E; e += 4) {
    int cnt = 0;
    for (int i = lane; i < nv; i += 64) {
      const uint4 q = reinterpret_cast<const uint4*>(smap)[(e * T >> 4) + i];
      *reinterpret_cast<uint4*>(map + (int64_t)e * Lpad + t0 + i * 16) = q;
      cnt += nonzero_bytes(q.x) + nonzero_bytes(q.y) + nonzero_bytes(q.z) + nonzero_bytes(q.w);
    }
    cnt = wave_sum(cnt);
    if (lane == 0) tilecnt[(int64_t)e * C + tile] = cnt;
  }
}

// Exclusive scan of each row of a [rows][C] count table (one workgroup per
// row): base[r][c] = r * row_offset + sum of counts[r][0..c).  total[r] gets
// the row sum when total is not null.
__global__ __launch_bounds__(256) void seg_scan(const int32_t* __restrict__ cnt, int C,
                                                int64_t row_offset, int32_t* __restrict__ base,
                                                int32_t* __restrict__ total) {
  __shared__ int scratch[4];
  const int r = blockIdx.x;
  int run = 0;
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int v = c < C ? cnt[(int64_t)r * C + c] : 0;
    int tot;
    const int inc = block256_incl_scan(v, scratch, &tot);
    if (c < C) base[(int64_t)r * C + c] = (int32_t)(r * row_offset + run + inc - v);
    run += tot;
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
  hipLaunchKernelGGL(seg_scan, dim3(rows), dim3(256), 0, s, cnt, C, row_offset, base, total);
}

// The streaming routing kernel handles E <= 64 with E % 4 == 0 and K <= 8
// (logits 16-byte aligned); it works on 256-token tiles.
static bool stream_path(int E, int K) { return E <= 64 && E % 4 == 0 && K <= 8; }

DispatchPlan plan_dispatch(int64_t L, int E, int K) {
  DispatchPlan p;
  // T is a power of two in [256, 1024] (the scatter kernel splits a
  // wavefront into T/16-lane row segments), with E * T <= 32 KB of LDS
  // where possible (E * T <= 64 KB always, since E <= 256).
  int T = 1024;
  while (T > 256 && E * T > 32768) T >>= 1;
  if (stream_path(E, K)) T = 256;
  p.T = T;
  p.C = (int)((L + T - 1) / T);
  p.Lpad = (int64_t)p.C * T;
  size_t o = 0;
  p.off_map = o;   o = align_up(o + (size_t)E * p.Lpad, 256);
  p.off_cnt = o;   o = align_up(o + (size_t)E * p.C * 4, 256);
  p.off_base = o;  o = align_up(o + (size_t)E * p.C * 4, 256);
  p.off_total = o; o = align_up(o + 256 * 4, 256);
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
    if (rows_ok && stream_path(E, K) && pl.T == 256) {
#define K1S(EBV, KV)                                                                         \
  hipLaunchKernelGGL((k1_route_map_stream<EBV, KV>), dim3(pl.C), dim3(256), 0, s, logits, L, E, \
                     pl.C, pl.Lpad, tei, gates, map, cnt)
#define K1S_K(EBV)                                                                           \
  switch (K) {                                                                               \
    case 1: K1S(EBV, 1); break;                                                              \
    case 2: K1S(EBV, 2); break;                                                              \
    case 3: K1S(EBV, 3); break;                                                              \
    case 4: K1S(EBV, 4); break;                                                              \
    case 5: K1S(EBV, 5); break;                                                              \
    case 6: K1S(EBV, 6); break;                                                              \
    case 7: K1S(EBV, 7); break;                                                              \
    default: K1S(EBV, 8); break;                                                             \
  }
      if (E <= 16) {
        K1S_K(16)
      } else if (E <= 32) {
        K1S_K(32)
      } else {
        K1S_K(64)
      }
#undef K1S_K
#undef K1S
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
    launch_seg_scan(cnt, E, pl.C, 0, base, total, s);
  }
  {
    LaunchTimer lt("dispatch_scatter", s);
    hipLaunchKernelGGL(k3_scatter, dim3(pl.C), dim3(256), 0, s, map, pl.Lpad, E, K, pl.T, pl.C,
                       base, total, eti, offsets, tim);
  }
  return hipGetLastError();
}

}  // namespace moe
