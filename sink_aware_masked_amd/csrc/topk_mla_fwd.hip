#include "common.hpp"
namespace attn {
hipError_t launch_topk_mla_bf16(const Params&, int, hipStream_t) { return hipErrorNotSupported; }
}
