// Host-side internal interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Brackets one kernel launch with timing events when kernel timing is on.
struct LaunchTimer {
  LaunchTimer(const char* name, hipStream_t s);
  ~LaunchTimer();
  int slot;
  hipStream_t stream;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Exclusive scan of each row of a [rows][C] int32 table:
// base[r][c] = r * row_offset + sum(cnt[r][0..c)); total[r] = row sum (if not null).
void launch_seg_scan(const int32_t* cnt, int rows, int C, int64_t row_offset, int32_t* base,
                     int32_t* total, hipStream_t s);

// ---------------------------------------------------------------- dispatch
struct DispatchPlan {
  int T;          // tokens per tile
  int C;          // tiles
  int64_t Lpad;   // C * T (row length of the token-expert map)
  bool stream;    // bit-form map (E <= 1024, K <= 8)
  int W;          // 64-bit mask words per token (bit form)
  int64_t NP;     // 64-token parts of the streaming router (per-part counts)
  size_t off_map, off_col, off_cnt, off_base, off_total, bytes;
};
DispatchPlan plan_dispatch(int64_t L, int E, int K);
hipError_t launch_dispatch(const DispatchPlan& pl, int64_t L, int E, int K, const float* logits,
                           int32_t* eti, int32_t* offsets, int32_t* tei, int32_t* tim,
                           float* gates, char* ws, hipStream_t s);

// ---------------------------------------------------------------- ffn
struct FfnDims {
  int64_t L;
  int d, h, E, K, dtype, act;
  bool recompute_g;  // no G buffer: G (gate * G) formed from A, B in L-row pieces
};

struct FfnPlan {
  int64_t R;
  int64_t route_tiles;   // upper bound of route-major M tiles
  int64_t pass_tiles;    // upper bound of M tiles per slot pass
  int64_t list_chunks;   // chunks of the slot-list builder
  size_t off_g, off_acc, off_slot, off_list, off_cnt, off_base, off_peoff, off_gatep, off_dgp;
  size_t off_tiles_route, off_tiles_pass, off_wt, off_zero, off_chunk, bytes;
  int n_chunk;           // expert groups of dW2 under recompute_g (at most 2K + 1)
};
FfnPlan plan_ffn(const FfnDims& dm, bool backward);

hipError_t launch_forward(const FfnPlan& pl, const FfnDims& dm, const void* x, const void* W1,
                          const void* W3, const void* W2, const int32_t* eti,
                          const int32_t* offsets, const int32_t* tim, const float* gates,
                          void* y, void* A, void* B, char* ws, hipStream_t s);

hipError_t launch_backward(const FfnPlan& pl, const FfnDims& dm, const void* dy, const void* x,
                           const void* W1, const void* W3, const void* W2, const int32_t* eti,
                           const int32_t* offsets, const int32_t* tim, const float* gates,
                           void* A, void* B, void* dx, void* dW1, void* dW3, void* dW2,
                           const int32_t* tei, float* dlogits, char* ws, hipStream_t s);

}  // namespace moe
