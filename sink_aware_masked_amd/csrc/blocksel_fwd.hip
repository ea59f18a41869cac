#include "common.hpp"
namespace attn {
hipError_t launch_blocksel_bf16(const Params&, int, hipStream_t) { return hipErrorNotSupported; }
}
