// Internal declarations shared by the host-side executor and the schedule
// generator (both are library code; nothing here is used by the oracle).
#pragma once

#include <vector>

#include "pps.h"

namespace pps {

enum { OP_F = PPS_OP_F, OP_B = PPS_OP_B, OP_W = PPS_OP_W };

struct Op3 {
    int kind;
    int mb;
    int chunk;
};

// Full op list of stage k (see pps_make_schedule).  Returns a PPS_* status.
int build_schedule(int P, int M, int k, int v, int kind, std::vector<pps_op>& out);

}  // namespace pps
