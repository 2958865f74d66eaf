// gla_bwd.hip -- chunkwise GLA backward (work in progress).
#include "prep.hpp"
namespace gla {
template <typename T, int DKP, int CP>
hipError_t launch_gla_bwd(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
#define GLA_BWD_INST(TT, D, C_) template hipError_t launch_gla_bwd<TT, D, C_>(const BwdParams&, hipStream_t);
#define GLA_BWD_INST_T(TT)                                                     \
  GLA_BWD_INST(TT, 32, 32) GLA_BWD_INST(TT, 32, 64) GLA_BWD_INST(TT, 32, 128)  \
  GLA_BWD_INST(TT, 64, 32) GLA_BWD_INST(TT, 64, 64) GLA_BWD_INST(TT, 64, 128)  \
  GLA_BWD_INST(TT, 128, 32) GLA_BWD_INST(TT, 128, 64) GLA_BWD_INST(TT, 128, 128) \
  GLA_BWD_INST(TT, 256, 32) GLA_BWD_INST(TT, 256, 64)
GLA_BWD_INST_T(bf16)
GLA_BWD_INST_T(float)
}  // namespace gla
