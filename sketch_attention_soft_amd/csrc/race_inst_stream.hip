// race_inst_stream.hip -- launch sequences of the RACE attention library
// instantiated for one row type and direction (race_host.h), compiled apart
// from the other race_inst_*.hip files so that the library builds in parallel.
#include "race_host.h"

namespace race_host {

RACE_STATE_ADD_INST(, bf16);
RACE_STATE_ADD_INST(, _Float16);
RACE_STREAM_INST(, bf16, race::SM_ADD);
RACE_STREAM_INST(, bf16, race::SM_DECODE);
RACE_STREAM_INST(, bf16, race::SM_READOUT);
RACE_STREAM_INST(, _Float16, race::SM_ADD);
RACE_STREAM_INST(, _Float16, race::SM_DECODE);
RACE_STREAM_INST(, _Float16, race::SM_READOUT);
RACE_STREAM_INST(, float, race::SM_ADD);
RACE_STREAM_INST(, float, race::SM_DECODE);
RACE_STREAM_INST(, float, race::SM_READOUT);

}  // namespace race_host
