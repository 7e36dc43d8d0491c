// Instances of the decode backward (Nq = 1) for the backward's head
// dimensions, 64 .. 1024 in steps of 64, and the group sizes it is built for:
// up to 4 query heads per kv head at D <= 512, up to 2 above (the registers
// of a wave hold q, dO and the dQ partial of every head of its group).
#include "dec_bwd.hpp"

namespace ffpa {
#define FFPA_DB(D, G)                                                              \
  template hipError_t launch_dec_bwd<D, false, G>(const DecBwdArgs&, hipStream_t); \
  template hipError_t launch_dec_bwd<D, true, G>(const DecBwdArgs&, hipStream_t);
#define FFPA_DB_LO(D) FFPA_DB(D, 1) FFPA_DB(D, 2) FFPA_DB(D, 4)
#define FFPA_DB_HI(D) FFPA_DB(D, 1) FFPA_DB(D, 2)
FFPA_DB_LO(64) FFPA_DB_LO(128) FFPA_DB_LO(192) FFPA_DB_LO(256)
FFPA_DB_LO(320) FFPA_DB_LO(384) FFPA_DB_LO(448) FFPA_DB_LO(512)
FFPA_DB_HI(576) FFPA_DB_HI(640) FFPA_DB_HI(704) FFPA_DB_HI(768)
FFPA_DB_HI(832) FFPA_DB_HI(896) FFPA_DB_HI(960) FFPA_DB_HI(1024)
#undef FFPA_DB_LO
#undef FFPA_DB_HI
#undef FFPA_DB
}  // namespace ffpa
