// libtaco kernels for INT8 codes (one translation unit per code format keeps
// each compilation small; see taco_kernels.hpp for the kernels).
#include "taco_kernels.hpp"

template struct taco_internal::Ops<taco_internal::Fmt::kInt8>;
