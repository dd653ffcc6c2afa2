// Measurement knobs that the kernels' launch planners read (process-global,
// atomic; defined in host.hip).
#pragma once

namespace w2a8 {

// Forced configuration of the pipelined MFMA GEMM (index into its table of
// configurations), or -1 for the automatic choice.
int gemm_pipe_force();
void set_gemm_pipe_force(int cfg);
constexpr int kGemmPipeConfigs = 10;

}  // namespace w2a8
