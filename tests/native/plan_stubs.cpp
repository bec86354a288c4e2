// Host-only stand-ins for the symbols libfd's device sources provide, so the
// planner (plan.cpp, api.cpp) links without the HIP kernels. The fuzzer always
// passes num_cus, so the occupancy queries and launches are never reached.
#include "fd_internal.h"
namespace fd {
int launch_merge(const MergeParams&, int, void*) { return 1; }
int launch_read_probe(const void*, long, unsigned int*, int, void*) { return 1; }
int launch_split_mfma(const SplitParams&, int, int, int, void*) { return 1; }
int launch_split_valu(const SplitParams&, int, int, int, int, void*) { return 1; }
int occupancy_split_mfma(int, int, int, int, int* o) { *o = 1; return 0; }
int occupancy_split_valu(int, int, int, int, int* o) { *o = 1; return 0; }
uint64_t* wg_stamp_records_for(int64_t) { return nullptr; }
}
