// HBM read-ceiling probe (read_probe.hip), launched by spec_hbm_read_probe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// `grid` workgroups of 4 waves, each wave writing 64 words of sink
// (grid * 256 <= SV_PROBE_SINK_WORDS).  Two workgroups per compute unit: with
// one, too few loads are in flight to reach the device's read rate (6.0
// against 6.8 TB/s on the pages of the 70B batch-256 workload).
constexpr int kProbeWgPerCu = 2;

void launch_hbm_read_probe(const void *k, const void *v, const int32_t *chunks, int64_t n, int chunk_bytes,
                           int64_t buffer_chunks, uint32_t *sink, int grid, hipStream_t stream);

}  // namespace sv
