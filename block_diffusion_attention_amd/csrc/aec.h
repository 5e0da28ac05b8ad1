// Normalized-entropy / AEC reduction over vocabulary logits: kernel arguments,
// the split of each row's vocabulary and the host-side launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdattn {

struct AecArgs {
  const void* logits;          // [N][row_stride], bf16 or fp32
  int64_t row_stride;          // elements
  int n_rows;                  // N
  int vocab;                   // V
  int nsplit;                  // workgroups per row
  int64_t chunk;               // vocabulary entries per split (multiple of the vector width)
  float* part;                 // nsplit > 1: [N][nsplit][3] partial (max, sum, weighted sum)
  float* lse;                  // [N] natural-log normalizer
  float* hbar;                 // [N] entropy / log V
  const uint8_t* unresolved;   // [N]
  const int32_t* state_rows;   // [S+1]
  int n_states;
  const int32_t* pair_next;    // [P]
  const float* pair_h_source;  // [P]
  const float* pair_weight;    // [P]
  int n_pairs;
  float rho;
  float gate_max;
  float* h_state;              // [S]
  float* loss;                 // [1]
  // backward
  const float* grad_loss;      // [1] upstream gradient of the loss
  float* state_grad;           // [S] workspace: dL/dH_state
  float* row_coef;             // [N] workspace: dL/dHbar_i / ln V (0 for rows outside the pairs)
  void* dlogits;               // [N][row_stride], the logits' type
};

// Workgroups per row: enough for ~2048 workgroups in all, each split at least
// kAecMinChunk entries.
constexpr int kAecMinChunk = 8192;

hipError_t launch_aec_entropy(const AecArgs& a, bool bf16, hipStream_t s);
hipError_t launch_aec_reduce(const AecArgs& a, hipStream_t s);
hipError_t launch_aec_grad_coef(const AecArgs& a, hipStream_t s);
hipError_t launch_aec_grad(const AecArgs& a, bool bf16, hipStream_t s);

}  // namespace bdattn
