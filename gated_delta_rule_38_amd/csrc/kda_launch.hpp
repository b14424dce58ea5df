// Host-side launchers of the gfx950 KDA kernels (defined in the .hip files).
#pragma once
#include <hip/hip_runtime.h>
#include "kda_device.hpp"

namespace kda {
// CHUNK kernel, one workgroup per chain / segment (x2 for the segment-build roles).
hipError_t launch_chunk(const ChunkParams &p, int D, bool fp32, int grid, bool stall, hipStream_t st);
// Pipelined CHUNK kernel (d = 128, bf16, 32-token chunks), one 512-thread workgroup per chain / segment.
hipError_t launch_chunk_pipe(const ChunkParams &p, int grid, bool stall, hipStream_t st);
// Debug-mode check of cu_seqlens: *flag = 0 when cu[0] == 0, cu non-decreasing, cu[N] == Ttot.
hipError_t launch_check_cu(const int32_t *cu, int32_t N, int64_t Ttot, int32_t *flag, hipStream_t st);
// Debug-mode range check of g: *flag = 1 when any element lies outside [c.lo, c.hi] or is NaN.
hipError_t launch_check_g(const CheckG &c, int32_t *flag, hipStream_t st);
// Debug-mode check of decode slots: *flag = 1 when two requests name the same slot in [0, P).
hipError_t launch_check_slots(const int32_t *idx, int32_t R, int32_t P, int32_t *flag, hipStream_t st);
// PREP kernel over `nvc` virtual chunks x H heads.
hipError_t launch_prep(const PrepParams &p, int nvc, hipStream_t st);
// COMBINE kernel over chains x D/16 value slabs.
hipError_t launch_combine(const CombineParams &p, int D, bool split, int chains, hipStream_t st);
// DECODE kernel over requests x heads x D/32 value slabs.
hipError_t launch_decode(const DecodeParams &p, int D, bool io_f32, bool state_bf16, hipStream_t st);
}  // namespace kda
