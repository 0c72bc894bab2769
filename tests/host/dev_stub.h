// Controls and records of the device stand-ins (dev_stub.cpp).
#pragma once
#include "fx_plan.h"

namespace stub {
struct Launch {
  const char* name = nullptr;
  const void* a = nullptr;
  const void* b = nullptr;
  const void* c = nullptr;
};
extern int alloc_fails;       // dev_alloc fails while nonzero
extern int launch_fails;      // every launcher returns this code
extern int decode_grid;       // what fx::decode_grid reports
extern bool scratch_missing;  // dev_static_scratch finds no array
extern Launch last;           // the most recent launch
extern int launches;          // launches so far
}  // namespace stub
