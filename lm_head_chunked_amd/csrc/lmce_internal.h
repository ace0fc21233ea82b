// Internal declarations shared by the host planner (lmce_api.hip) and the
// device kernels (lmce_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmce {

constexpr int kStatusLabel = 1;   // asynchronous flag: a label was out of range
constexpr int kTile = 128;        // rows of h / W in one logit tile
constexpr int kStageK = 64;       // hidden-size granularity of the main loop

// First 256 bytes of the workspace.
struct WsHeader {
  int n_valid;   // rows whose label is not ignore_index (and is in range)
  int status;    // 0 or kStatusLabel
  int pad[62];
};

struct FwdArgs {
  const uint16_t* h;
  const uint16_t* W;
  const int64_t* labels;
  int64_t L, H, V, ignore_index;
  int chunk_rows;       // rows per schedule chunk
  int tiles_per_chunk;  // ceil(chunk_rows / 128)
  int n_chunks;         // ceil(L / chunk_rows)
  int segments;         // vocabulary segments swept by separate workgroups
  int vtiles;           // ceil(V / 128)
  int vtiles_per_seg;   // ceil(vtiles / segments)
  WsHeader* hdr;
  float* zlabel;        // [L] logit of each row's label
  float* part_m;        // [segments][L] running max per row and segment
  float* part_s;        // [segments][L] sum of exp(z - max) per row and segment
  float* block_sum;     // [ceil(L/256)] per-block nll sums
};

struct BwdArgs {
  const uint16_t* h;
  const uint16_t* W;
  const int64_t* labels;
  const float* lse;
  const float* grad_loss;
  const uint16_t* hT;   // [H][Lpad] transposed h, zero past L
  const uint16_t* WT;   // [H][Vpad] transposed W, zero past V
  int64_t L, H, V, ignore_index, Lpad, Vpad;
  int vtiles;
  WsHeader* hdr;
  float* dh;
  float* dW;
};

hipError_t launch_count_labels(const int64_t* labels, int64_t L, int64_t V, int64_t ignore_index, WsHeader* hdr,
                               hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, float* loss_out, float* lse_out, hipStream_t st);
hipError_t launch_transpose(const void* in, int64_t R, int64_t C, void* out, int64_t Rpad, hipStream_t st);
hipError_t launch_bwd_dh(const BwdArgs& a, int hs, hipStream_t st);
hipError_t launch_bwd_dW(const BwdArgs& a, int hs, hipStream_t st);

}  // namespace lmce
