// Launchers of the GPU kernels (defined in the .hip sources), stubbed out for
// the host-only sanitizer builds; calling one aborts.
#include <cstdlib>

#include "../../expert_cache_ffn_amd/csrc/ecf_internal.h"

namespace ecf {
int launch_router_logits(const ecf_shape &, const void *, const void *, int, float *, hipStream_t) { std::abort(); }
int launch_route(const ecf_shape &, const float *, int, const RouteOut &, hipStream_t) { std::abort(); }
int launch_decode_gateup(const ecf_shape &, const ExpertTables &, const RouteOut &, const void *, int, float *,
                         hipStream_t) { std::abort(); }
bool down_combine1_ok(const ecf_shape &, int) { return false; }
bool gateup_route1_ok(const ecf_shape &, int) { return false; }
int launch_decode_gateup_route1(const ecf_shape &, const ExpertTables &, const float *, const void *, const RouteOut &,
                                float *, hipStream_t) { std::abort(); }
int launch_decode_down_combine1(const ecf_shape &, const ExpertTables &, const RouteOut &, const float *, const float *,
                                float *, void *, hipStream_t) { std::abort(); }
int launch_decode_down(const ecf_shape &, const ExpertTables &, const RouteOut &, const float *, int, float *,
                       hipStream_t) { std::abort(); }
int launch_prefill_gemm1(const ecf_shape &, const ExpertTables &, const RouteOut &, const void *, int, uint16_t *,
                         hipStream_t) { std::abort(); }
int launch_prefill_gemm2(const ecf_shape &, const ExpertTables &, const RouteOut &, const uint16_t *, int, float *,
                         hipStream_t) { std::abort(); }
int launch_combine(const ecf_shape &, const ExpertTables &, const RouteOut &, const float *, int, const float *,
                   const float *, float *, void *, hipStream_t) { std::abort(); }
}  // namespace ecf
