// Internal interface of the matrix-core throughput probe (mfma_probe.hip) for the C-ABI layer
// (lard_api.cpp).  Not installed; not part of the public ABI.
#pragma once

namespace lard {

// Enqueue the probe (lard_probe_mfma): a hipError_t value, 0 on success.
int launch_probe_mfma(bool vector_work, int iters, int workgroups, float* sink, void* stream);

}  // namespace lard
