// placeholder, replaced by the decay-separable state scan kernels
#include "lrs_internal.h"
