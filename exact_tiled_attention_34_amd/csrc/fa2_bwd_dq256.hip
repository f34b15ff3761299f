// The dQ kernel at head dimension 256, compiled as a unit of its own (see
// launch_bwd_dq_d256 in fa2_bwd.hip): the same source, with only that
// launcher defined.
#define FA2_DQ256_UNIT 1
#include "fa2_bwd.hip"
