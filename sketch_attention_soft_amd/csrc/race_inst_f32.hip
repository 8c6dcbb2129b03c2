// race_inst_f32.hip -- launch sequences of the RACE attention library
// instantiated for one row type and direction (race_host.h), compiled apart
// from the other race_inst_*.hip files so that the library builds in parallel.
#include "race_host.h"

namespace race_host {

RACE_FWD_INST(, float);
RACE_BWD_INST(, float);
RACE_SPLIT_FWD_INST(, float);
RACE_SPLIT_BWD_INST(, float);

}  // namespace race_host
