// igc_launch.hip -- kernel instantiations: launch<KIND, VAR> of igc_host.hpp
// for the (kind, variant) pairs of IGC_LAUNCH_KINDS.  The build
// compiles this file once per pair with -DIGC_LAUNCH_UNIT=<n>, so the kinds
// compile in parallel; without the define it instantiates every pair.
#include "igc_host.hpp"

namespace igc_host {

#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 0
template int launch<igc::KIND_F16_GEMM, 0>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 1
template int launch<igc::KIND_F16_CONV, 0>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 2
template int launch<igc::KIND_F16_CONV_C64, 0>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 3
template int launch<igc::KIND_U8I8_GEMM, 0>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 4
template int launch<igc::KIND_U8I8_GEMM, 1>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 5
template int launch<igc::KIND_U8I8_GEMM, 2>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 6
template int launch<igc::KIND_U8I8_GEMM, 3>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 7
template int launch<igc::KIND_U8I8_CONV, 0>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 8
template int launch<igc::KIND_U8I8_CONV, 1>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 9
template int launch<igc::KIND_U8I8_CONV, 2>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 10
template int launch<igc::KIND_U8I8_CONV, 3>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 11
template int launch<igc::KIND_U8I8_GEMM, 4>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 12
template int launch<igc::KIND_U8I8_GEMM, 5>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 13
template int launch<igc::KIND_U8I8_GEMM, 6>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 14
template int launch<igc::KIND_U8I8_GEMM, 7>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 15
template int launch<igc::KIND_U8I8_CONV, 4>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 16
template int launch<igc::KIND_U8I8_CONV, 5>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 17
template int launch<igc::KIND_U8I8_CONV, 6>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 18
template int launch<igc::KIND_U8I8_CONV, 7>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 19
template int launch<igc::KIND_F16_CONV, 8>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 20
template int launch<igc::KIND_F16_CONV_C64, 8>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 21
template int launch<igc::KIND_U8I8_GEMM, 20>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 22
template int launch<igc::KIND_U8I8_GEMM, 21>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 23
template int launch<igc::KIND_U8I8_CONV, 20>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 24
template int launch<igc::KIND_U8I8_CONV, 21>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 25
template int launch<igc::KIND_F16_GEMM, 32>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 26
template int launch<igc::KIND_F16_CONV, 32>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 27
template int launch<igc::KIND_F16_CONV_C64, 32>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 28
template int launch<igc::KIND_F16_CONV, 40>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 29
template int launch<igc::KIND_F16_CONV_C64, 40>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 30
template int launch<igc::KIND_U8I8_GEMM, 32>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 31
template int launch<igc::KIND_U8I8_GEMM, 33>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 32
template int launch<igc::KIND_U8I8_GEMM, 34>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 33
template int launch<igc::KIND_U8I8_GEMM, 35>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 34
template int launch<igc::KIND_U8I8_CONV, 32>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 35
template int launch<igc::KIND_U8I8_CONV, 33>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 36
template int launch<igc::KIND_U8I8_CONV, 34>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif
#if !defined(IGC_LAUNCH_UNIT) || IGC_LAUNCH_UNIT == 37
template int launch<igc::KIND_U8I8_CONV, 35>(const igc::Params&, const Plan&, bool, hipStream_t);
#endif

}  // namespace igc_host
