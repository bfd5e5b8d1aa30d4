// Included first (-include) by the MemorySanitizer build of the tree driver:
// every LDS array of a tree kernel is marked uninitialised when a workgroup
// starts, then the workgroup's lanes meet at a barrier before using it.
#pragma once
#include <sanitizer/msan_interface.h>
#define BT_LDS_POISON(x)                              \
  do {                                                \
    __msan_poison((void*)&(x), sizeof(x));            \
    __syncthreads();                                  \
  } while (0)
