// Host-only stand-ins for the HIP launchers of libkda.so, so that the C-ABI
// host layer (kda_api.cpp: argument checks, workspace sizing, failure
// injection) can be built with g++ and AddressSanitizer and run on a machine
// without a GPU. Every launcher reports that no device is present, which is
// what the real library reports there; none touches the memory it is given.
#include "kda_launch.h"

namespace kda {

hipError_t launch_chunk_fwd(const ChunkFwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_chunk_prep(const ChunkFwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_chunk_state_pass(const ChunkFwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_chunk_transition(const ChunkFwdArgs&, float*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_affine_scan(const float*, const float*, const float*, float*, int64_t, int64_t,
                              int64_t, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_step(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_spec(const SpecArgs&, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_spec_commit_verify(const SpecArgs&, const SpecPrefix&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t noalloc_scratch(void**) { return hipErrorNoDevice; }

}  // namespace kda
